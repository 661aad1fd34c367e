/*
 * moe_ffn.h - C ABI of the MI355X (gfx950) routed MoE expert FFN library.
 *
 * The library implements the expert half of a mixture-of-experts layer with
 * a live-row contract: top-k routing, a scatter into a per-expert aligned
 * ("grouped") layout described by int32 expert end offsets, two grouped MX
 * GEMMs around a fused SiLU*up + FP8 quantisation that touches live rows
 * only, a weighted top-k combine, and a sparse per-(token, slot) GEMV path
 * for small decode batches.
 *
 * Page keys used in the citations below:
 *   [LIVE]   "Blackwell FP4 MoE: live-row boundary" (review of the vLLM
 *            live-row change)
 *   [SGL]    "Blackwell DeepGEMM FusedMoE (sglang)" (SGLang v0.5.21
 *            DeepGEMM FusedMoE walkthrough)
 *   [XSERV]  "Phase 20: Sparse MoE Decode" (xserv sparse decode design)
 *   [KIMI]   "Kimi-K3 on SM120 FlashInfer MXFP4" (Kimi-K3 SM120 experiment)
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * - Pointers are DEVICE pointers unless stated otherwise. Every tensor is
 *   dense, row-major, with the shape given in brackets. bf16 values are
 *   passed as uint16_t bit patterns; E4M3 and packed E2M1 as uint8_t.
 * - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *   enqueues work on it and returns; nothing synchronises and nothing is read
 *   back to the host, so a chain of calls can be captured in a HIP graph.
 *   Grid sizes depend only on the integer arguments, never on routed counts.
 * - Ownership: the caller allocates and owns all memory. The library never
 *   allocates, frees, retains or aliases a pointer ([SGL] section 3.6.1's
 *   use-after-free lesson). Outputs must not overlap inputs.
 * - Live-row contract ([LIVE] sections 2-3): inside the grouped layout the
 *   rows of local expert e are [start_e, end_e) with
 *       start_0 = 0, start_e = align_up(end_{e-1}, A), end_e = start_e + count_e.
 *   Only expert_ends[E_local] is stored; consumers rebuild start_e from the
 *   previous end. Producers write live rows only and consumers read live
 *   rows only: rows in alignment gaps and the capacity tail are never read or
 *   written, so they keep whatever the caller put there. Device-side end
 *   values are clamped to [0, M_cap] before use, so corrupt metadata cannot
 *   cause out-of-bounds accesses.
 * - Packed UE8M0 scale layout ("MN-major"): for a K-wide FP8 matrix with one
 *   E8M0 byte per 32 columns, word c of row r sits at scales[c * M_cap + r]
 *   (shape [K/128][M_cap] int32) and holds the bytes of column groups
 *   4c..4c+3 in byte 0..3 (little endian) ([SGL] section 2.4.1 and
 *   Appendix A: K-groups packed four per int32, MN-major).
 * - Errors: every argument is validated on the host before anything is
 *   enqueued; a failed check returns a negative MOE_ERR_* code with no side
 *   effects. MOE_ERR_LAUNCH reports a failed kernel launch. There is no
 *   silent fallback path. Zero-sized work (T == 0, E_local == 0) returns
 *   MOE_OK without enqueuing anything.
 * - The library holds no state and is thread-safe, with one exception:
 *   moe_scatter_endpoints_noalloc keeps a fixed device array (its scratch)
 *   on every GPU it runs on, for the life of the process.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 14

enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,          /* a required pointer is NULL */
    MOE_ERR_SHAPE = -2,         /* a size is negative, zero where it may not be, or too large */
    MOE_ERR_ALIGN = -3,         /* a size is not a multiple of what the layout requires */
    MOE_ERR_CAPACITY = -4,      /* M_cap cannot hold the worst-case grouped layout */
    MOE_ERR_UNSUPPORTED = -5,   /* an enum or parameter value this build does not support */
    MOE_ERR_LAUNCH = -6,        /* a kernel launch failed (hipGetLastError) */
    MOE_ERR_WORKSPACE = -7,     /* workspace missing or smaller than moe_scatter_workspace_bytes() */
    MOE_ERR_SCRATCH = -8,       /* the sizes need more than a no-alloc entry point's static scratch */
    MOE_ERR_DEVICE = -9         /* the current device or its static scratch could not be queried */
};

enum moe_score_fn {
    MOE_SCORE_SOFTMAX = 0,       /* top-k of logits, softmax over the selected k */
    MOE_SCORE_SIGMOID_BIAS = 1   /* top-k of sigmoid(logit)+bias, weights sigmoid renormalised */
};

enum moe_weight_format {
    MOE_W_FP8_PER_EXPERT = 0,    /* E4M3 weights [E_local, N, K] + float scale per expert */
    MOE_W_MXFP4_G32 = 1          /* E2M1 pairs [E_local, N, K/2] + E8M0 byte per 32 columns */
};

/* Version of this ABI (MOE_ABI_VERSION). A binding must refuse a library
 * whose version differs from the header it was written against. */
int moe_abi_version(void);

/* Static, never-NULL text for a status code. */
const char* moe_status_string(int status);

/* ------------------------------------------------------------------------
 * moe_route - top-k expert selection and routing weights.
 * [SGL] section 1 (gate scores, top-k, combine weights); [XSERV] section 1
 * (router -> topk_softmax); [KIMI] Phase 1 call chain (sigmoid scores, the
 * correction bias only selects experts, weights gathered from the unbiased
 * sigmoid and renormalised).
 *
 *   logits          fp32 [T, E]
 *   score_fn        MOE_SCORE_SOFTMAX: ids = the k largest logits;
 *                     weights = softmax over the selected k.
 *                   MOE_SCORE_SIGMOID_BIAS: s = sigmoid(logit) rounded to
 *                     fp32, key = fl32(s + correction_bias[e]); ids = the k
 *                     largest keys; weights = s_sel / sum(s_sel).
 *   correction_bias fp32 [E]; required for SIGMOID_BIAS, must be NULL otherwise
 *   topk_ids        int32 [T, k] out; slot 0 is the best; equal keys go to
 *                   the lower expert index
 *   topk_weights    fp32 [T, k] out
 * Limits: 1 <= k <= min(E, 32), 1 <= E <= 1024. Logits must be finite.
 * ------------------------------------------------------------------------ */
int moe_route(const float* logits, int T, int E, int k, int score_fn,
              const float* correction_bias, int32_t* topk_ids, float* topk_weights,
              void* stream);

/* Bytes of device workspace moe_scatter_endpoints needs for these sizes. */
size_t moe_scatter_workspace_bytes(int T, int k, int E_local);

/* ------------------------------------------------------------------------
 * moe_scatter_endpoints - grouped-layout scatter with int32 expert ends and
 * the per-32 FP8 quantisation of each routed token row.
 * [LIVE] section 2 (endpoint recurrence; the scatter writes the int32
 * endpoints in its existing step, no device-to-host read of counts);
 * [SGL] section 2.2.4 (compact layout: per-token-group FP8 quant with packed
 * UE8M0 scales, scatter into aligned expert segments) and Appendix C
 * (row <-> token-slot map).
 *
 *   topk_ids     int32 [T, k]; a route is local when
 *                e = id - expert_start lies in [0, E_local); other ids
 *                (negative, or another GPU's experts) are skipped
 *   A            alignment of each expert segment's start (>= 1)
 *   M_cap        rows of the grouped buffers; must satisfy
 *                M_cap >= T*k + E_local*A and M_cap % 4 == 0
 *   x            bf16 [T, H] token activations; H % 128 == 0
 *   expert_ends  int32 [E_local] out: end_e of the recurrence above
 *   route_row    int32 [T*k] out: for local route r = t*k+s, start_e plus the
 *                number of earlier local routes (smaller r) of the same
 *                expert; -1 for non-local routes
 *   xq           u8 [M_cap, H] out: E4M3 codes of x[t] in row route_row[r];
 *                live rows only
 *   xs           int32 [H/128][M_cap] out: packed UE8M0 scales (MN-major);
 *                live rows only
 *   workspace    device scratch of at least moe_scatter_workspace_bytes()
 * Quantisation of each 32-column group v: amax = max|v|, q = fl32(amax/448),
 * b = UE8M0 round-up of q ([SGL] section 2.3.2 bit rule), code_i =
 * e4m3_rne(v_i / 2^(b-127)). Limits: E_local <= 1024, k <= 32.
 * ------------------------------------------------------------------------ */
int moe_scatter_endpoints(const int32_t* topk_ids, int T, int k, int expert_start, int E_local,
                          int A, int M_cap, const uint16_t* x, int H,
                          int32_t* expert_ends, int32_t* route_row, uint8_t* xq, int32_t* xs,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_scatter_endpoints_noalloc - moe_scatter_endpoints without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments, outputs, limits and errors as moe_scatter_endpoints
 * (group-32 recipe), minus workspace / workspace_bytes. The per-(token block,
 * expert) counters live in a static device array of 135,168 bytes instead
 * (32,768 counters plus 1,024 expert starts, the most any call within the
 * limits needs; sizes that would need more return MOE_ERR_SCRATCH before
 * anything is enqueued). The array exists once per GPU, for the life of the
 * process; its address on the current device is looked up on the first call
 * on that device (MOE_ERR_DEVICE if that fails), so `stream` must belong to
 * the current device. The call allocates nothing. Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race on it and must be
 * ordered by the caller. Contents left by an earlier call are never read:
 * each call writes every counter before reading it.
 * ------------------------------------------------------------------------ */
int moe_scatter_endpoints_noalloc(const int32_t* topk_ids, int T, int k, int expert_start,
                                  int E_local, int A, int M_cap, const uint16_t* x, int H,
                                  int32_t* expert_ends, int32_t* route_row, uint8_t* xq,
                                  int32_t* xs, void* stream);

/* ------------------------------------------------------------------------
 * moe_pack_mx_weights - one-time, load-time relayout of MXFP4 expert weights
 * (codes and E8M0 scales) into the fragment-ordered form the grouped GEMMs
 * stream.
 * [SGL] section 2.1 (weight preparation runs once at load time so that the
 * run-time GEMM never touches the checkpoint layout) and 2.1.2 (weights and
 * scales are rewritten into the layout the GEMM kernel consumes).
 *
 *   w               u8 [E, N, K/2]: two E2M1 codes per byte, low nibble =
 *                   even column (checkpoint layout)
 *   w_scale         u8 [E, N, K/32]: E8M0 byte of columns [32j, 32j+32)
 *   w_packed        u8, E*N*K/2 bytes, out: for column block cb = n/16 and
 *                   k-step ks = k/128 a 1 KB chunk at ((e*N/16 + cb)*K/128 + ks)*1024
 *                   whose 16 bytes at lane*16 are bytes [64ks + 16(lane/16), +16)
 *                   of row 16cb + lane%16
 *   w_scale_packed  u8, E*(K/128)*(N/64)*256 bytes (= E*N*K/32), out: for
 *                   k-step ks, group q of 4 column blocks and lane l (0..63)
 *                   a 4-byte word at (((e*K/128 + ks)*N/64 + q)*64 + l)*4
 *                   whose byte b is the E8M0 byte of group 4ks + l/16 of row
 *                   16(4q + b) + l%16 (a wave's 4 column blocks of one step
 *                   are 256 contiguous bytes)
 * Pure data movement (bit-exact). Requires K % 128 == 0, N % 64 == 0,
 * E <= 65535. The caller owns all four buffers; the packed buffers are what
 * moe_grouped_gemm1 / moe_grouped_gemm2 take.
 * ------------------------------------------------------------------------ */
int moe_pack_mx_weights(const uint8_t* w, const uint8_t* w_scale, int E, int N, int K,
                        uint8_t* w_packed, uint8_t* w_scale_packed, void* stream);

/* ------------------------------------------------------------------------
 * moe_pack_mx_weights_gateup - moe_pack_mx_weights for the fused GEMM1 +
 * activation path: the same code and scale layouts, with the column blocks
 * of w13 reordered so that each 256-column group holds the gate blocks of
 * one 128-column slice of h and their up blocks, interleaved two by two.
 * [SGL] section 2.1 (load-time weight preparation into the layout the
 * kernel consumes) and 2.4 (activation and quantisation fused).
 *
 *   w13, w13_scale  as for moe_pack_mx_weights with N = 2I, K = H
 *   w_packed, w_scale_packed  out, sizes as for moe_pack_mx_weights; packed
 *                   column block p = 16t + 4c + k holds source block
 *                   8t + 2c + k (gate) for k < 2 and I/16 + 8t + 2c + k - 2
 *                   (up) for k >= 2
 * Requires I % 128 == 0 and the conditions of moe_pack_mx_weights.
 * ------------------------------------------------------------------------ */
int moe_pack_mx_weights_gateup(const uint8_t* w13, const uint8_t* w13_scale, int E, int I,
                               int H, uint8_t* w_packed, uint8_t* w_scale_packed, void* stream);

/* ------------------------------------------------------------------------
 * moe_grouped_gemm1_act_quant - moe_grouped_gemm1 followed by
 * moe_act_quant_liverows in one kernel: the gate/up products of each live
 * row are rounded to bf16 (the gateup values moe_grouped_gemm1 would
 * store), then SiLU(gate)*up is formed and quantised to E4M3 + UE8M0
 * exactly as moe_act_quant_liverows does on those bf16 values, so hq and
 * hs are byte-identical to the two-call path; gateup never reaches memory.
 * [SGL] section 2.4 (act + quant fused, gate/up read once); [LIVE]
 * sections 1-3 (live rows only, padding untouched).
 *
 *   xq, xs, expert_ends, E_local, A, M_cap, H, I  as for moe_grouped_gemm1
 *   w13_gateup_packed, w13_gateup_scale_packed  moe_pack_mx_weights_gateup
 *                of w13 and its scales
 *   clamp_limit  as for moe_act_quant_liverows
 *   hq, hs       as for moe_act_quant_liverows (out, live rows only)
 * Requires I % 128 == 0, M_cap * I < 2^31 and the conditions of
 * moe_grouped_gemm1.
 * ------------------------------------------------------------------------ */
int moe_grouped_gemm1_act_quant(const uint8_t* xq, const int32_t* xs, const int32_t* expert_ends,
                                int E_local, int A, int M_cap, int H, int I,
                                const uint8_t* w13_gateup_packed,
                                const uint8_t* w13_gateup_scale_packed, float clamp_limit,
                                uint8_t* hq, int32_t* hs, void* stream);

/* ------------------------------------------------------------------------
 * moe_grouped_gemm1 - gate/up projection of every live row with its expert's
 * MXFP4 w13, on scaled MX MFMA.
 * [SGL] sections 2.3 and 3.3 (contiguous grouped FP8 x FP4 GEMM: lhs
 * (all_tokens, K) fp8 + scale, rhs (E, 2I, K//2) packed fp4 + scale,
 * out (all_tokens, 2I) bf16); [LIVE] section 2 (FC1 consumes the endpoints);
 * [KIMI] checkpoint contract (w13 holds contiguous [gate; up] halves).
 *
 *   xq, xs       as produced by moe_scatter_endpoints (K = H)
 *   expert_ends  int32 [E_local]
 *   w13_packed, w13_scale_packed
 *                moe_pack_mx_weights of w13 u8 [E_local, 2I, H/2] (two E2M1
 *                codes per byte, low nibble = even column; rows 0..I-1 gate,
 *                I..2I-1 up) and its E8M0 scales u8 [E_local, 2I, H/32]
 *   gateup       bf16 [M_cap, 2I] out: live rows only,
 *                gateup[r, n] = bf16_rne(sum_k xq*2^(xs-127) * w13*2^(s-127))
 *                accumulated in fp32
 * Requires H % 128 == 0, I % 64 == 0, E_local <= 1024.
 * ------------------------------------------------------------------------ */
int moe_grouped_gemm1(const uint8_t* xq, const int32_t* xs, const int32_t* expert_ends,
                      int E_local, int A, int M_cap, int H, int I,
                      const uint8_t* w13_packed, const uint8_t* w13_scale_packed,
                      uint16_t* gateup, void* stream);

/* ------------------------------------------------------------------------
 * moe_act_quant_liverows - SiLU(gate)*up + FP8/UE8M0 quantisation of live
 * rows only.
 * [LIVE] sections 1-3 (the activation kernel takes the same endpoints,
 * loops only over [start, end) of each expert and leaves padding
 * unwritten); [SGL] section 2.4 (act and quant fused: read bf16 once, write
 * fp8 + scale once; silu_mul_keep_fp32: SiLU stays fp32; default-branch
 * clamp: up on both sides, gate from above only).
 *
 *   gateup       bf16 [M_cap, 2I] (row = [gate I | up I])
 *   clamp_limit  <= 0 or +inf: no clamp; otherwise L > 0 and exactly
 *                representable in bf16: g = min(g, L), u = min(max(u,-L), L)
 *   hq           u8 [M_cap, I] out: E4M3 codes, live rows only
 *   hs           int32 [I/128][M_cap] out: packed UE8M0 scales, live rows only
 * Per element: s = sigmoid(g) rounded to fp32; h = fl32(fl32(g*s) * u); then
 * the per-32 quantisation of moe_scatter_endpoints on h.
 * Requires I % 128 == 0, M_cap % 4 == 0, E_local <= 1024, M_cap <= 3,145,728,
 * M_cap * I * 4 < 2^31 (else MOE_ERR_SHAPE).
 * ------------------------------------------------------------------------ */
int moe_act_quant_liverows(const uint16_t* gateup, const int32_t* expert_ends, int E_local,
                           int A, int M_cap, int I, float clamp_limit,
                           uint8_t* hq, int32_t* hs, void* stream);

/* ------------------------------------------------------------------------
 * moe_act_quant_liverows_situ - moe_act_quant_liverows with the SiTU
 * activation instead of SiLU.
 * [SGL] section 2.4.1, situ branch (gate' = b_s tanh(g/b_s) sigmoid(g),
 * up' = b_l tanh(u/b_l), then gate' * up' and the group quantisation);
 * [KIMI] (Kimi-K3's reference formula with b_s = 4, b_l = 25).
 *
 *   gateup, expert_ends, E_local, A, M_cap, I, hq, hs
 *                as for moe_act_quant_liverows
 *   situ_beta, situ_linear_beta  must be 4.0 and 25.0 (the function tables
 *                are built for these; anything else is MOE_ERR_UNSUPPORTED)
 * Per element: t = 4 tanh(g/4), s = sigmoid(g), v = 25 tanh(u/25), each
 * rounded to fp32; h = fl32(fl32(t*s) * v); then the per-32 quantisation
 * of moe_scatter_endpoints on h. No clamp. Same limits as
 * moe_act_quant_liverows.
 * ------------------------------------------------------------------------ */
int moe_act_quant_liverows_situ(const uint16_t* gateup, const int32_t* expert_ends, int E_local,
                                int A, int M_cap, int I, float situ_beta, float situ_linear_beta,
                                uint8_t* hq, int32_t* hs, void* stream);

/* ------------------------------------------------------------------------
 * moe_grouped_gemm2 - down projection of every live row with its expert's
 * MXFP4 w2.
 * [SGL] section 2.5.1 (second contiguous grouped GEMM; the activation
 * recipe follows K = I); [LIVE] section 2 (FC2 consumes the endpoints).
 *
 *   hq, hs       as produced by moe_act_quant_liverows (K = I)
 *   w2_packed, w2_scale_packed
 *                moe_pack_mx_weights of w2 u8 [E_local, H, I/2] and its E8M0
 *                scales u8 [E_local, H, I/32]
 *   down         bf16 [M_cap, H] out: live rows only
 * Requires I % 128 == 0, H % 128 == 0, E_local <= 1024.
 * ------------------------------------------------------------------------ */
int moe_grouped_gemm2(const uint8_t* hq, const int32_t* hs, const int32_t* expert_ends,
                      int E_local, int A, int M_cap, int I, int H,
                      const uint8_t* w2_packed, const uint8_t* w2_scale_packed,
                      uint16_t* down, void* stream);

/* ------------------------------------------------------------------------
 * Natural-weight forms: moe_grouped_gemm1, moe_grouped_gemm2 and
 * moe_grouped_gemm1_act_quant taking the weights in their checkpoint layout
 * instead of the packed one, so that no load-time preparation is needed.
 * [SGL] sections 2.3 and 3.3 (the contiguous grouped GEMM's rhs is
 * (E, N, K//2) packed fp4 with (E, N, K//32) E8M0 scales); [KIMI] checkpoint
 * contract (w13 rows [gate; up]).
 *
 *   w13, w13_scale  u8 [E_local, 2I, H/2] (two E2M1 codes per byte, low
 *                   nibble = even column; rows 0..I-1 gate, I..2I-1 up) and
 *                   u8 [E_local, 2I, H/32] (E8M0)
 *   w2, w2_scale    u8 [E_local, H, I/2] and u8 [E_local, H, I/32]
 * Every other argument, requirement, output and error as in the packed
 * forms, whose results these reproduce bit for bit (the same products are
 * summed in the same order; only where the weight bytes are read from
 * differs). The packed forms stay the faster path for repeated calls.
 * ------------------------------------------------------------------------ */
int moe_grouped_gemm1_natural(const uint8_t* xq, const int32_t* xs, const int32_t* expert_ends,
                              int E_local, int A, int M_cap, int H, int I, const uint8_t* w13,
                              const uint8_t* w13_scale, uint16_t* gateup, void* stream);
int moe_grouped_gemm2_natural(const uint8_t* hq, const int32_t* hs, const int32_t* expert_ends,
                              int E_local, int A, int M_cap, int I, int H, const uint8_t* w2,
                              const uint8_t* w2_scale, uint16_t* down, void* stream);
int moe_grouped_gemm1_act_quant_natural(const uint8_t* xq, const int32_t* xs,
                                        const int32_t* expert_ends, int E_local, int A,
                                        int M_cap, int H, int I, const uint8_t* w13,
                                        const uint8_t* w13_scale, float clamp_limit,
                                        uint8_t* hq, int32_t* hs, void* stream);

/* ------------------------------------------------------------------------
 * Group-128 activation recipe: the four entry points below are the group-32
 * ones above with activations quantised per 128 columns instead of 32.
 * [SGL] overview (table of quantised data types) and section 2.1.3 (the
 * MXFP4-experts recipe quantises activations per (1,128), weights per
 * (1,32)); section 2.2.4 (with UE8M0 scales the activation scales are int32
 * words packing 4 consecutive groups, column-major, ceil(K/128/4) words per
 * token). Per 128-column group: amax, the
 * UE8M0 round-up of amax/448 and the e4m3 codes exactly as in the group-32
 * forms, with 128 in place of 32.
 *
 *   scales       int32 [ceil(K/512), M_cap]: byte j of word c is the group of
 *                columns [512c + 128j, +128); bytes of groups past K are 0
 *                (K = H for the scatter and GEMM1 inputs, I for the
 *                act-quant output and the GEMM2 input)
 *   codes        as in the group-32 forms
 * The GEMMs apply a group's scale to each of its four 32-column blocks (the
 * weights keep their per-32 E8M0 scales). Same arguments, requirements,
 * ownership and errors as moe_scatter_endpoints, moe_grouped_gemm1,
 * moe_act_quant_liverows and moe_grouped_gemm2 respectively, except the
 * scale layout. moe_grouped_gemm1_act_quant_g128 is
 * moe_grouped_gemm1_act_quant with group-128 input scales xs and group-128
 * output scales hs ([SGL] section 2.4: act + quant fused); its hq and hs are
 * byte-identical to moe_grouped_gemm1_g128 followed by
 * moe_act_quant_liverows_g128.
 * ------------------------------------------------------------------------ */
int moe_scatter_endpoints_g128(const int32_t* topk_ids, int T, int k, int expert_start,
                               int E_local, int A, int M_cap, const uint16_t* x, int H,
                               int32_t* expert_ends, int32_t* route_row, uint8_t* xq, int32_t* xs,
                               void* workspace, size_t workspace_bytes, void* stream);
int moe_grouped_gemm1_g128(const uint8_t* xq, const int32_t* xs, const int32_t* expert_ends,
                           int E_local, int A, int M_cap, int H, int I,
                           const uint8_t* w13_packed, const uint8_t* w13_scale_packed,
                           uint16_t* gateup, void* stream);
int moe_act_quant_liverows_g128(const uint16_t* gateup, const int32_t* expert_ends, int E_local,
                                int A, int M_cap, int I, float clamp_limit, uint8_t* hq,
                                int32_t* hs, void* stream);
int moe_grouped_gemm1_act_quant_g128(const uint8_t* xq, const int32_t* xs,
                                     const int32_t* expert_ends, int E_local, int A, int M_cap,
                                     int H, int I, const uint8_t* w13_gateup_packed,
                                     const uint8_t* w13_gateup_scale_packed, float clamp_limit,
                                     uint8_t* hq, int32_t* hs, void* stream);
int moe_grouped_gemm2_g128(const uint8_t* hq, const int32_t* hs, const int32_t* expert_ends,
                           int E_local, int A, int M_cap, int I, int H,
                           const uint8_t* w2_packed, const uint8_t* w2_scale_packed,
                           uint16_t* down, void* stream);

/* ------------------------------------------------------------------------
 * Masked slab layout: the five entry points below run the chain on an
 * [E_local, m_pad, K] buffer in which every local expert owns a fixed block
 * of m_pad rows, in place of the aligned layout.
 * [SGL] section 2.2.4 (standard masked pre-permute: bucket the routes per
 * expert into fixed slabs and quantise them in one step, producing masked_m,
 * the real row count of each expert), section 2.3.2 and section 3.2 (masked
 * grouped GEMM: lhs (E, m, K) fp8 with (E, m, G/4) int32 UE8M0 scales in
 * MN-major memory, only the first masked_m[e] rows of expert e computed,
 * out (E, m, N) bf16), section 2.4.2 (varlen act-quant bounded by masked_m)
 * and section 2.5.2 (masked GEMM2 into (E, m, K)).
 *
 * Layout: expert e's rows are [e*m_pad, e*m_pad + masked_m[e]); the rest of
 * its block is padding that no call reads or writes. A route's row inside
 * its block is its rank among the expert's local routes in flattened route
 * order t*k+s (as in the aligned layout). Scale words are MN-major per
 * expert: word c of row j of expert e at scales[(e*W + c)*m_pad + j], with
 * W = K/128 words per row (shape [E_local][K/128][m_pad] int32, bytes as in
 * the aligned layout). m_pad must be a multiple of 4 and E_local*m_pad <
 * 2^31; every other requirement is that of the aligned form.
 *
 * Capacity: the pages size m_pad so that no expert overflows (m_pad >= the
 * token count T always suffices, since a token's k ids are distinct). A
 * route whose rank inside its expert reaches m_pad is not placed: its
 * route_row is -1 and masked_m[e] = min(count_e, m_pad), so the combine
 * leaves it out. masked_m values are clamped into [0, m_pad] by every
 * consumer. The pages' expected_m (a kernel-selection hint) has no
 * counterpart: the GEMMs schedule from masked_m on the device.
 *
 * moe_scatter_masked: moe_scatter_endpoints into the slab (same quantisation,
 *   same workspace: moe_scatter_workspace_bytes(T, k, E_local));
 *   masked_m int32 [E_local] out; route_row int32 [T*k] out (e*m_pad + rank,
 *   or -1); xq u8 [E_local*m_pad, H] out; xs int32 [E_local][H/128][m_pad] out.
 *   m_pad >= 4 when E_local > 0.
 * moe_grouped_gemm1_masked: moe_grouped_gemm1 on the slab; gateup bf16
 *   [E_local*m_pad, 2I] out.
 * moe_act_quant_masked: moe_act_quant_liverows (SiLU, optional clamp) on the
 *   slab; hq u8 [E_local*m_pad, I] out; hs int32 [E_local][I/128][m_pad] out.
 *   E_local*m_pad <= 3,145,728 as for moe_act_quant_liverows.
 * moe_grouped_gemm1_act_quant_masked: moe_grouped_gemm1_act_quant on the
 *   slab (hq, hs as moe_act_quant_masked writes them).
 * moe_grouped_gemm2_masked: moe_grouped_gemm2 on the slab; down bf16
 *   [E_local*m_pad, H] out. moe_combine then takes rows = down, n_rows =
 *   E_local*m_pad and row_of_slot = route_row.
 * Group-32 activation recipe only.
 * ------------------------------------------------------------------------ */
int moe_scatter_masked(const int32_t* topk_ids, int T, int k, int expert_start, int E_local,
                       int m_pad, const uint16_t* x, int H, int32_t* masked_m,
                       int32_t* route_row, uint8_t* xq, int32_t* xs, void* workspace,
                       size_t workspace_bytes, void* stream);
int moe_grouped_gemm1_masked(const uint8_t* xq, const int32_t* xs, const int32_t* masked_m,
                             int E_local, int m_pad, int H, int I, const uint8_t* w13_packed,
                             const uint8_t* w13_scale_packed, uint16_t* gateup, void* stream);
int moe_act_quant_masked(const uint16_t* gateup, const int32_t* masked_m, int E_local, int m_pad,
                         int I, float clamp_limit, uint8_t* hq, int32_t* hs, void* stream);
int moe_grouped_gemm1_act_quant_masked(const uint8_t* xq, const int32_t* xs,
                                       const int32_t* masked_m, int E_local, int m_pad, int H,
                                       int I, const uint8_t* w13_gateup_packed,
                                       const uint8_t* w13_gateup_scale_packed, float clamp_limit,
                                       uint8_t* hq, int32_t* hs, void* stream);
int moe_grouped_gemm2_masked(const uint8_t* hq, const int32_t* hs, const int32_t* masked_m,
                             int E_local, int m_pad, int I, int H, const uint8_t* w2_packed,
                             const uint8_t* w2_scale_packed, uint16_t* down, void* stream);

/* ------------------------------------------------------------------------
 * moe_combine - unpermute and weighted top-k sum.
 * [SGL] section 2.6.1 (post_reorder: per token, fp32 sum over slots whose
 * destination row is >= 0 of weight * row, times routed_scaling_factor);
 * [XSERV] section 3 (skip non-local slots, never multiply them by zero).
 *
 *   rows         bf16 [n_rows, H]
 *   row_of_slot  int32 [T*k]; entries outside [0, n_rows) (e.g. -1) are skipped
 *   topk_weights fp32 [T, k]
 *   out          bf16 [T, H] out:
 *                acc = 0; for s = 0..k-1: if row valid: acc = fl32(acc + fl32(w*v));
 *                out = bf16_rne(fl32(acc * routed_scale))  (no fused multiply-add)
 * Requires H % 8 == 0, k <= 32.
 * ------------------------------------------------------------------------ */
int moe_combine(const uint16_t* rows, int64_t n_rows, const int32_t* row_of_slot,
                const float* topk_weights, int T, int k, int H, float routed_scale,
                uint16_t* out, void* stream);

/* ------------------------------------------------------------------------
 * moe_sparse_gemv - decode-time expert GEMV that reads only the experts the
 * router picked, each selected expert's weights once per call.
 * [XSERV] sections 2-3 (M=1 is bandwidth-bound; each block reads topk_ids
 * on the device and exits when the expert is not local; bias fused in the
 * epilogue acc*w_scale + bias; non-local slots are not written; gate_up and
 * down share one kernel, x shared by the slots of a token for gate_up,
 * per-slot activations for down) and section 4 (used for <= 8 tokens);
 * [KIMI] mismatch matrix (GPT-OSS GLU parameters alpha=1.702, beta=1,
 * limit=7).
 *
 *   act          bf16: [T, K] when act_per_slot == 0, [T*k, K] when 1
 *   topk_ids     int32 [T, k]; local window [expert_start, expert_start+E_local)
 *   wfmt         MOE_W_FP8_PER_EXPERT: w u8 [E_local, N, K] E4M3,
 *                  w_scale float [E_local]
 *                MOE_W_MXFP4_G32: w u8 [E_local, N, K/2], w_scale u8
 *                  [E_local, N, K/32] (E8M0)
 *   bias         bf16 [E_local, N] or NULL
 *   y[n]         = bf16_rne(fl32(acc*w_scale) + bias[n]) (FP8) or
 *                  bf16_rne(acc + bias[n]) (MXFP4), acc accumulated in fp32
 *   glu          0: out bf16 [T*k, N] holds y.
 *                1: out bf16 [T*k, N/2] holds, for j < N/2,
 *                   bf16(g' * sigmoid(glu_alpha*g') * (u' + glu_beta)) with
 *                   g = y[j], u = y[j+N/2] (already rounded to bf16),
 *                   g' = min(g, glu_limit), u' = clamp(u, -glu_limit, glu_limit)
 *                   (glu_limit <= 0: no clamp).
 *                2: the GLU on load: act is the per-slot gate/up output of
 *                   a glu = 0 call, bf16 [T*k, 2K] (act_per_slot must be 1),
 *                   and the activation element j of slot q is the bf16 value
 *                   of the formula above with g = act[q, j], u = act[q, K+j];
 *                   out bf16 [T*k, N] holds y. A glu = 1 gate_up call
 *                   followed by a glu = 0 down call gives the same bytes as
 *                   a glu = 0 gate_up call followed by a glu = 2 down call.
 *   out          row t*k+s is written only when slot (t,s) is local
 *   slot_row     int32 [T*k] out or NULL: t*k+s when local, else -1
 * Requires K % 32 == 0 (FP8: K % 16 == 0 suffices), K <= 8192, N % 2 == 0
 * when glu == 1, 1 <= T*k <= 64, E_local <= 1024; glu outside 0..2, or
 * glu == 2 with act_per_slot == 0, is MOE_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------ */
int moe_sparse_gemv(const uint16_t* act, int act_per_slot, const int32_t* topk_ids, int T, int k,
                    int expert_start, int E_local, int N, int K, int wfmt, const uint8_t* w,
                    const void* w_scale, const uint16_t* bias, int glu, float glu_alpha,
                    float glu_beta, float glu_limit, uint16_t* out, int32_t* slot_row,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
