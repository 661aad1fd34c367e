// moe_sparse_gemv: decode-time expert GEMV that reads only the experts the
// router picked, on gfx950.
//
// "Phase 20: Sparse MoE Decode", sections 2-3: at M = 1 the expert GEMV is
// bound by weight bytes, so only routed experts are read; each block reads
// topk_ids on the device and leaves at once (block-uniformly, before any
// LDS or barrier) when its expert is not local; bias and the per-expert
// scale are fused into the epilogue; non-local slots are never written.
// Section 4: the path serves batches of at most 8 tokens.
//
// Differences from the page's kernel: blocks are keyed by slot, but only
// the first slot (in t*k+s order) of each distinct local expert does work,
// and it computes every slot routed to that expert, one after the other, so
// each selected expert's weights are read once per call instead of once per
// slot. A thread's chunk is 16 bytes of a weight row: 16 FP8 weights, or 32
// E2M1 weights (one E8M0 group). For FP8 a block owns 8 weight rows (4 gate +
// 4 up rows when the GLU is fused, else 8 output columns) and its 256 threads
// split K; for MXFP4, whose rows are half as long, a block owns 16 rows in two
// groups of 8, each split over 128 threads. Every chunk a thread needs is
// loaded at once, with the bias of its epilogue column; the matching
// activations are read straight from memory into registers. Chunks are
// converted to exact bf16 pairs and dotted in fp32; the partial sums are
// folded inside each wave with DPP adds and across the waves of a row group
// through LDS in a fixed order. With the GLU fused, the GLU is applied to the
// bf16-rounded gate and up results before the single bf16 store. With the
// GLU applied on load instead (GLU_LOAD), the activation rows are the
// per-slot gate/up outputs of the first GEMV ([T*k, 2K]: gate then up) and
// each activation element is the bf16 rounding of the GLU of its gate and
// up values, formed as the chunk is read; the results equal those of the
// fused form, whose stored activation is that same bf16 value.
#include <cmath>
#include <type_traits>

#include "common.h"

namespace moe {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / 64;
constexpr int kGemvRows = 8;          // weight rows per row group (FP8: the block; GLU: 4 gate + 4 up)
constexpr int kGemvMaxSlots = 64;     // T*k
constexpr int kGemvSlotBatch = 1;     // slots accumulated together (one: the fewer
                                      // registers, the more waves per SIMD, which
                                      // measured faster than sharing conversions)
constexpr int kGemvMaxCh = 2;         // 16-byte chunks per thread and row (K <= 8192)

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float glu_apply(float g, float u, float alpha, float beta, float limit) {
  if (limit > 0.f) {
    g = fminf(g, limit);
    u = fminf(fmaxf(u, -limit), limit);
  }
  const float sig = 1.0f / (1.0f + expf(-alpha * g));
  return g * sig * (u + beta);
}

// Sum over the wave, left in lane 63: inclusive scan inside each 16-lane row
// (row_shr 1, 2, 4, 8), then rows 1 and 3 add row 0's and row 2's totals
// (row_bcast:15) and rows 2 and 3 add lane 31 (row_bcast:31). Fixed order.
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  auto step = [](float x, auto ctrl, auto rmask) -> float {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value,
                                                          decltype(rmask)::value, 0xF, false));
  };
  v = step(v, std::integral_constant<int, 0x111>{}, std::integral_constant<int, 0xF>{});
  v = step(v, std::integral_constant<int, 0x112>{}, std::integral_constant<int, 0xF>{});
  v = step(v, std::integral_constant<int, 0x114>{}, std::integral_constant<int, 0xF>{});
  v = step(v, std::integral_constant<int, 0x118>{}, std::integral_constant<int, 0xF>{});
  v = step(v, std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xA>{});
  v = step(v, std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xC>{});
  return v;
}

// 16 FP8 weights (16 bytes) -> 8 exact bf16 pairs
__device__ __forceinline__ void fp8x16_to_bf16(const v4i raw, v2bf* wp) {
  const uint32_t d[4] = {(uint32_t)raw.x, (uint32_t)raw.y, (uint32_t)raw.z, (uint32_t)raw.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    wp[2 * q + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[q], 1.0f, false);
    wp[2 * q + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[q], 1.0f, true);
  }
}
// 32 E2M1 weights (16 bytes, low nibble first) -> 16 exact bf16 pairs
__device__ __forceinline__ void fp4x32_to_bf16(const v4i raw, v2bf* wp) {
  const uint32_t d[4] = {(uint32_t)raw.x, (uint32_t)raw.y, (uint32_t)raw.z, (uint32_t)raw.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    wp[4 * q + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[q], 1.0f, 0);
    wp[4 * q + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[q], 1.0f, 1);
    wp[4 * q + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[q], 1.0f, 2);
    wp[4 * q + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[q], 1.0f, 3);
  }
}

// A thread's chunk is 16 bytes of a row: 16 FP8 weights, or 32 E2M1 weights
// (one E8M0 scale group). A row group of threads covers K: all 256 threads
// for FP8; 128 for MXFP4, whose rows are half as long, so that a block
// holds 2 row groups of 8 rows (16 rows, about the bytes of FP8's 8).
template <bool MXFP4, bool GLU, int CH, bool GLU_LOAD>
__global__ __launch_bounds__(kGemvThreads) void sparse_gemv_kernel(
    const uint16_t* __restrict__ act, int act_per_slot, const int32_t* __restrict__ ids, int T,
    int k, int expert_start, int E_local, int N, int K, const uint8_t* __restrict__ W,
    const void* __restrict__ w_scale, const uint16_t* __restrict__ bias, float alpha,
    float beta, float limit, uint16_t* __restrict__ out, int32_t* __restrict__ slot_row) {
  constexpr int kTPR = MXFP4 ? 128 : 256;            // threads per row group
  constexpr int kRG = kGemvThreads / kTPR;           // row groups per block
  constexpr int kWPG = kTPR / 64;                    // waves per row group
  constexpr int kRows = kGemvRows * kRG;             // weight rows per block
  constexpr int kWpc = MXFP4 ? 32 : 16;              // weights per chunk
  __shared__ float s_red[kGemvWaves][kGemvSlotBatch][kGemvRows];

  const int q = blockIdx.y;  // flattened slot t*k+s
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wid / kWPG;                        // this thread's row group
  const int t = tid % kTPR;                          // its place in the group
  const int nq = T * k;      // <= 64: one id per lane
  // every wave reads all slot ids at once; the same ballots in every wave
  // give the duplicate test and the list of slots routed to this expert
  const int my_id = lane < nq ? ids[lane] : INT32_MIN;
  const int id = __shfl(my_id, q, 64);
  const int e = id - expert_start;
  const bool local = e >= 0 && e < E_local;
  if (blockIdx.x == 0 && tid == 0 && slot_row) slot_row[q] = local ? q : -1;
  if (!local) return;  // block-uniform, before any LDS use or barrier
  const uint64_t same = __ballot(my_id == id);
  // the first slot of each distinct local expert does the work
  if (same & ((1ull << q) - 1ull)) return;   // block-uniform

  const int n_out = GLU ? N / 2 : N;
  constexpr int kOuts = GLU ? kRows / 2 : kRows;     // output columns per block
  const int col0 = blockIdx.x * kOuts;
  const size_t row_bytes = MXFP4 ? (size_t)K / 2 : (size_t)K;
  const int nch = K / kWpc;            // chunks per row
  const uint8_t* We = W + (size_t)e * N * row_bytes;
  const float fp8_scale = MXFP4 ? 1.f : reinterpret_cast<const float*>(w_scale)[e];
  const uint8_t* Ws = MXFP4 ? reinterpret_cast<const uint8_t*>(w_scale) + (size_t)e * N * (K / 32)
                            : nullptr;
  // weight row of block row rr (clamped into range; columns past n_out are
  // computed and never stored); with the GLU, rows [0, kOuts) are gate rows
  // and [kOuts, 2 kOuts) the matching up rows
  auto row_of = [&](int rr) {
    if (GLU) return min(col0 + (rr % kOuts), n_out - 1) + (rr < kOuts ? 0 : N / 2);
    return min(col0 + rr, N - 1);
  };

  // the bias of this thread's epilogue column(s), fetched before the
  // weights so that its latency is hidden; read unpredicated (without a bias,
  // from the weight bytes, which are longer, and then not used)
  const uint16_t* bsrc = bias ? bias : reinterpret_cast<const uint16_t*>(W);
  uint16_t bpre[GLU ? 2 : 1];
#pragma unroll
  for (int hf = 0; hf < (GLU ? 2 : 1); ++hf)
    bpre[hf] = bsrc[(size_t)e * N + row_of(tid % kOuts + hf * kOuts)];

  // every weight chunk of this thread goes out first (unpredicated: a
  // thread past the last chunk reads the last one and does not use it)
  v4i raw[kGemvRows][CH];
  float gsc[MXFP4 ? kGemvRows : 1][CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int ch = min(t + kTPR * j, nch - 1);
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
      const int row = row_of(grp * kGemvRows + r);
      raw[r][j] = __builtin_nontemporal_load(
          reinterpret_cast<const v4i*>(We + (size_t)row * row_bytes + (size_t)ch * 16));
      if constexpr (MXFP4) gsc[r][j] = e8m0_value(Ws[(size_t)row * (K / 32) + ch]);
    }
  }

  for (uint64_t rest = same; rest;) {
    // the next batch of this expert's slots
    int p[kGemvSlotBatch];
    int S = 0;
#pragma unroll
    for (int b = 0; b < kGemvSlotBatch; ++b) {
      p[b] = -1;
      if (rest) {
        p[b] = __ffsll((unsigned long long)rest) - 1;
        rest &= rest - 1ull;
        S = b + 1;
      }
    }
    float acc[kGemvSlotBatch][kGemvRows];
#pragma unroll
    for (int b = 0; b < kGemvSlotBatch; ++b)
#pragma unroll
      for (int r = 0; r < kGemvRows; ++r) acc[b][r] = 0.f;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int ch = t + kTPR * j;
      const bool valid = ch < nch;
      const int chc = min(ch, nch - 1);
      // this chunk's activations of each slot of the batch
      v2bf av[kGemvSlotBatch][kWpc / 2];
#pragma unroll
      for (int b = 0; b < kGemvSlotBatch; ++b) {
        const int arow = p[b] < 0 ? 0 : (act_per_slot ? p[b] : p[b] / k);
        if constexpr (GLU_LOAD) {
          // gate at [arow, chunk], up K columns later; each pair -> bf16(glu)
          const uint16_t* gp = act + (size_t)arow * (2 * (size_t)K) + (size_t)chc * kWpc;
          const v4i* g4p = reinterpret_cast<const v4i*>(gp);
          const v4i* u4p = reinterpret_cast<const v4i*>(gp + K);
#pragma unroll
          for (int v = 0; v < kWpc / 8; ++v) {
            const v4i g4 = g4p[v], u4 = u4p[v];
            const uint32_t gw[4] = {(uint32_t)g4.x, (uint32_t)g4.y, (uint32_t)g4.z, (uint32_t)g4.w};
            const uint32_t uw[4] = {(uint32_t)u4.x, (uint32_t)u4.y, (uint32_t)u4.z, (uint32_t)u4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float lo = glu_apply(bf16_to_f32((uint16_t)(gw[i] & 0xFFFFu)),
                                         bf16_to_f32((uint16_t)(uw[i] & 0xFFFFu)), alpha, beta, limit);
              const float hi = glu_apply(bf16_to_f32((uint16_t)(gw[i] >> 16)),
                                         bf16_to_f32((uint16_t)(uw[i] >> 16)), alpha, beta, limit);
              const uint32_t packed = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
              av[b][4 * v + i] = __builtin_bit_cast(v2bf, packed);
            }
          }
        } else {
          const v4i* ap = reinterpret_cast<const v4i*>(act + (size_t)arow * K + (size_t)chc * kWpc);
#pragma unroll
          for (int v = 0; v < kWpc / 8; ++v) {
            const v4i a4 = ap[v];
            // components copied out first: a bit cast of a vector component
            // expression reads the vector's first component
            const int w4[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) av[b][4 * v + i] = __builtin_bit_cast(v2bf, w4[i]);
          }
        }
      }
      if (valid) {
#pragma unroll
        for (int r = 0; r < kGemvRows; ++r) {
          // converted per batch, row by row (only one row's pairs live)
          v4i rw = raw[r][j];
          asm volatile("" : "+v"(rw));
          v2bf wp[kWpc / 2];
          if constexpr (MXFP4) fp4x32_to_bf16(rw, wp);
          else fp8x16_to_bf16(rw, wp);
#pragma unroll
          for (int b = 0; b < kGemvSlotBatch; ++b) {
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < kWpc / 2; ++i)
              part = __builtin_amdgcn_fdot2_f32_bf16(wp[i], av[b][i], part, false);
            if constexpr (MXFP4) acc[b][r] = fmaf(part, gsc[r][j], acc[b][r]);
            else acc[b][r] = acc[b][r] + part;
          }
        }
      }
    }
    // fold: inside the wave (DPP, lane 63), then the group's waves in order
#pragma unroll
    for (int b = 0; b < kGemvSlotBatch; ++b)
#pragma unroll
      for (int r = 0; r < kGemvRows; ++r) {
        const float v = wave_sum_to_lane63(acc[b][r]);
        if (lane == 63) s_red[wid][b][r] = v;
      }
    __syncthreads();
    // epilogue: thread (b, c) owns output column c of slot b
    if (tid < kGemvSlotBatch * kOuts) {
      const int b = tid / kOuts, c = tid % kOuts;
      const int j = col0 + c;
      if (b < S && j < n_out) {
        float y[2];
#pragma unroll
        for (int hf = 0; hf < (GLU ? 2 : 1); ++hf) {
          const int rr = c + hf * kOuts;                 // block row
          const int g0 = rr / kGemvRows, r = rr % kGemvRows;
          float tot = s_red[g0 * kWPG][b][r];
#pragma unroll
          for (int w = 1; w < kWPG; ++w) tot += s_red[g0 * kWPG + w][b][r];
          const float bv = bias ? bf16_to_f32(bpre[hf]) : 0.f;
          const float yv = MXFP4 ? __fadd_rn(tot, bv) : __fadd_rn(__fmul_rn(tot, fp8_scale), bv);
          y[hf] = bf16_to_f32((uint16_t)f32_to_bf16_bits(yv));
        }
        const float v = GLU ? glu_apply(y[0], y[1], alpha, beta, limit) : y[0];
        out[(size_t)p[b] * n_out + j] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
    if (rest) __syncthreads();   // s_red is reused by the next batch
  }
}

}  // namespace moe

extern "C" int moe_sparse_gemv(const uint16_t* act, int act_per_slot, const int32_t* topk_ids,
                               int T, int k, int expert_start, int E_local, int N, int K, int wfmt,
                               const uint8_t* w, const void* w_scale, const uint16_t* bias, int glu,
                               float glu_alpha, float glu_beta, float glu_limit, uint16_t* out,
                               int32_t* slot_row, void* stream) {
  using namespace moe;
  if (T < 0 || k < 1 || E_local < 0 || E_local > 1024 || N <= 0 || K <= 0) return MOE_ERR_SHAPE;
  if ((long long)T * k > kGemvMaxSlots) return MOE_ERR_SHAPE;
  if (wfmt != MOE_W_FP8_PER_EXPERT && wfmt != MOE_W_MXFP4_G32) return MOE_ERR_UNSUPPORTED;
  if (glu < 0 || glu > 2) return MOE_ERR_UNSUPPORTED;
  // GLU on load: the activation is the per-slot gate/up rows [T*k, 2K]
  if (glu == 2 && act_per_slot != 1) return MOE_ERR_UNSUPPORTED;
  if (K % (wfmt == MOE_W_MXFP4_G32 ? 32 : 16) != 0) return MOE_ERR_ALIGN;
  if (K % 8 != 0) return MOE_ERR_ALIGN;
  if (glu == 1 && N % 2 != 0) return MOE_ERR_ALIGN;
  if (act_per_slot != 0 && act_per_slot != 1) return MOE_ERR_UNSUPPORTED;
  const bool mx = wfmt == MOE_W_MXFP4_G32;
  // FP8: 16 weights per thread chunk over 256 threads; MXFP4: 32 over 128
  const int chunks_per_thread = mx ? (K / 32 + 127) / 128 : (K / 16 + kGemvThreads - 1) / kGemvThreads;
  if (chunks_per_thread > kGemvMaxCh) return MOE_ERR_SHAPE;  // K <= 8192
  if (T == 0) return MOE_OK;
  if (!act || !topk_ids || !w || !w_scale || !out) return MOE_ERR_NULL;
  const int n_out = glu == 1 ? N / 2 : N;
  const int rows_per_block = mx ? 2 * kGemvRows : kGemvRows;
  const int outs_per_block = glu == 1 ? rows_per_block / 2 : rows_per_block;
  dim3 grid((n_out + outs_per_block - 1) / outs_per_block, T * k);
  hipStream_t st = (hipStream_t)stream;
#define MOE_GEMV_LAUNCH(MX, G, CHN, GL)                                                        \
  hipLaunchKernelGGL((sparse_gemv_kernel<MX, G, CHN, GL>), grid, dim3(kGemvThreads), 0, st, act, \
                     act_per_slot, topk_ids, T, k, expert_start, E_local, N, K, w, w_scale, bias, \
                     glu_alpha, glu_beta, glu_limit, out, slot_row)
#define MOE_GEMV_CH(MX, G, GL)                       \
  switch (chunks_per_thread) {                       \
    case 1: MOE_GEMV_LAUNCH(MX, G, 1, GL); break;    \
    default: MOE_GEMV_LAUNCH(MX, G, 2, GL); break;   \
  }
  if (mx && glu == 1) MOE_GEMV_CH(true, true, false)
  else if (mx && glu == 2) MOE_GEMV_CH(true, false, true)
  else if (mx) MOE_GEMV_CH(true, false, false)
  else if (glu == 1) MOE_GEMV_CH(false, true, false)
  else if (glu == 2) MOE_GEMV_CH(false, false, true)
  else MOE_GEMV_CH(false, false, false)
#undef MOE_GEMV_CH
#undef MOE_GEMV_LAUNCH
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
