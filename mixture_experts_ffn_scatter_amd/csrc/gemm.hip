// moe_grouped_gemm1 / moe_grouped_gemm2: grouped MX GEMMs over the live rows
// of the aligned expert layout, on gfx950 scaled MFMA; and
// moe_pack_mx_weights, the load-time weight preparation they consume.
//
//   out[m, n] = sum_k X[m, k] * W_e[n, k]      for m in [start_e, end_e)
//
// X is E4M3 with one UE8M0 byte per 32 columns (packed MN-major, four per
// int32), W_e is E2M1 with one E8M0 byte per 32 columns ("Blackwell DeepGEMM
// FusedMoE (sglang)", sections 2.3 / 2.5 / 3.3 and 3.8: contiguous grouped
// FP8 x FP4 GEMM with (1,32) weight scales; here the activation recipe is
// (1,32) as well). "Blackwell FP4 MoE: live-row boundary", section 2: both
// GEMMs take the int32 expert ends; rows outside [start_e, end_e) are
// neither read nor written.
//
// Mapping onto V_MFMA_SCALE_F32_16X16X128_F8F6F4 (lane layout measured on
// gfx950 with a one-instruction probe): the weight tile is the A operand
// (16 output columns x 128 k, E2M1, 16 bytes per lane) and the activation
// tile the B operand (128 k x 16 rows, E4M3, 32 bytes per lane). With
// g = lane/16, an E2M1 operand holds k-slice [32g, 32g+32) of row lane%16 in
// order (low nibble first), while an E4M3 operand holds k [16g, 16g+16) in
// its first four dwords and k [64+16g, 64+16g+16) in the last four. The
// E8M0 scale of row r and 32-wide k-block b is read from lane r + 16b. The
// 16x16 fp32 result gives lane l four consecutive output columns of row
// l%16, stored as one 8-byte bf16 write.
//
// Weight preparation (once, at load time; "Blackwell DeepGEMM FusedMoE
// (sglang)", section 2.1: weights are rearranged into the layout the GEMM
// consumes, so that the run-time GEMM never touches the checkpoint layout):
// codes are stored in MFMA fragment order, one contiguous 1 KB chunk per
// (16-column block, 128-wide k-step), and scales per (k-step, group of 4
// column blocks) as 64 lane words (byte c of lane l's word: the byte lane l
// of the MFMA needs for column block 4q + c), so that one k-step of a
// 256-column tile's scales is one contiguous 1 KB block and a wave reads
// its 4 column blocks' scales as one word.
//
// Work decomposition. An item is (expert, n-tile of 256 columns, m-chunk of
// up to 128 live rows); its cost grows with its live row blocks (a full
// chunk takes about 1.6 times a one-block chunk). Chunks are ranked by
// cost, full ones first, then partial ones by row blocks descending. The
// full chunks are cut into 8 contiguous runs, one per XCD (block b runs on
// XCD b % 8), so the chunks of a many-chunk expert share its weights in few
// L2s; the partial chunks are dealt to the XCDs in snake order. Every chunk
// goes with all its n-tiles, so the items of a chunk share its activations
// in one XCD's L2. An XCD lists its items chunk-major, costliest first, and
// its blocks take them in snake order over rounds, so a block with a costly
// item in one round gets a cheap one in the next. The ranking is rebuilt
// inside every block from expert_ends (a block-wide scan and count), so
// the grid depends only on host-known sizes and no count is read back.
//
// Data path. Every operand travels global -> LDS by the buffer-to-LDS
// transfer of gfx950 (no register staging) into a ring of 4 stages of one
// k-step each (activations, weights and both scale sets: 33.5 KB a stage).
// A step issues the transfers of the step 3 ahead (continuing into the next
// item of the block), so 3 steps of loads are always in flight; each wave
// waits for its own transfers of the current stage with an exact count and
// one barrier publishes the stage. The 8 waves form 2 row groups x 4
// column groups; wave (rg, cg) owns rows [64 rg, +64) x columns [64 cg, +64)
// of the tile, so per step it reads 4 weight and 4 activation fragments
// (12 KB of LDS for 16 MFMAs) and issues up to 16 MFMAs, reading the
// activation fragments two row blocks ahead of the MFMAs that consume them.
// Every wave issues the same 5 transfers a step (2 weight chunks, 2 halves
// of an activation row block, one dword of scales), so the step body has no
// per-wave branch, and they go out in pairs after each row block's MFMAs
// (pinned by scheduling barriers) rather than queueing at the step's start
// ahead of them. Steps are software-pipelined across the barrier: a step
// waits, synchronises and reads the next step's weight fragments, scale
// words and first activation fragments before its own last row block's
// MFMAs, so the matrix cores keep working while the block synchronises.
// Loads use buffer resources whose range ends at the last live row (or
// column): lanes past it read zeros without touching memory, so
// padding rows are never read.
#include "common.h"

#include <cstring>
#include <type_traits>

namespace moe {
namespace gemm_act {
// sigma(g) for every bf16 g (the activation kernel's table, generated at
// build time; a private copy for the fused GEMM1 epilogue, read through L2)
#define MOE_SIGMOID_TABLE_STORAGE static __device__ const __attribute__((aligned(16)))
#include "sigmoid_table.inc"
#undef MOE_SIGMOID_TABLE_STORAGE
}  // namespace gemm_act
}  // namespace moe
#include "sigmoid_lookup.h"

namespace moe {

constexpr int kGemmBN = 256;       // columns per item (16 blocks of 16)
constexpr int kGemmBM = 128;       // rows per item (8 blocks of 16)
constexpr int kGemmStages = 4;     // LDS ring depth (k-steps)
constexpr int kGemmMB = 4;         // row blocks per wave (MFMA)
constexpr int kGemmMaxE = 1024;
constexpr uint32_t kOob = 0x80000000u;  // buffer offset past any range: reads zero, no traffic

// The wave layout of a 128 x 256 tile: 8 waves in 2 row groups x 4 column
// groups, each 64 rows x 64 columns (16 MFMAs and 12 KB of LDS reads per
// step; accumulators in VGPRs).
struct Gemm8 {
  static constexpr int waves = 8;
  static constexpr int threads = 64 * waves;
  static constexpr int CB = 4;                             // column blocks per wave
  static constexpr int CG = kGemmBN / 16 / CB;             // column groups of waves
  static constexpr int RG = kGemmBM / 16 / kGemmMB;        // row groups of waves
  static constexpr int dma_cb = kGemmBN / 16 / waves;      // weight chunks a wave moves per step
  static constexpr int dma_xr = kGemmBM / 16 / waves;      // activation row blocks a wave moves
  static constexpr int ops = dma_cb + 2 * dma_xr + 1;      // transfers a wave issues per step
  static_assert(RG * CG == waves, "wave grid");
  static_assert(dma_cb * waves == kGemmBN / 16 && dma_xr * waves == kGemmBM / 16,
                "transfers split evenly over the waves");
};
constexpr int kGemmThreads = Gemm8::threads;

// One LDS stage: everything one k-step of a 128 x 256 tile reads.
//   x[mb][h]: activations of rows 16mb.. in B-fragment order (lane l: 16 bytes
//             of row 16mb + l%16 at k 64h + 16(l/16))
//   w[cb]:    weight codes of column block cb in A-fragment order
//   xs[row]:  the row's 4 UE8M0 bytes (k-blocks 0..3 of the step)
//   ws:       the tile's weight scales: for column-block group q (4 blocks)
//             lane l's 4 E8M0 bytes at 256 q + 4 l (byte c: block 4q + c)
struct __attribute__((aligned(16))) GemmStage {
  uint8_t x[kGemmBM / 16][2][1024];
  uint8_t w[kGemmBN / 16][1024];
  uint32_t xs[kGemmBM];
  uint8_t ws[64][kGemmBN / 16];
};
constexpr int kOffW = kGemmBM / 16 * 2 * 1024;
constexpr int kOffXs = kOffW + kGemmBN / 16 * 1024;
constexpr int kOffWs = kOffXs + kGemmBM * 4;
static_assert(sizeof(GemmStage) == kOffWs + kGemmBN / 16 * 64, "stage layout");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // raw buffer (stride 0); word 3 as for every gfx9 raw buffer
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// Buffer-to-LDS transfers: lane l's 16 (or 4) bytes at buffer offset voff
// land at LDS byte address m0 + 16 l (or m0 + 4 l). Lanes past the buffer's
// range write zeros and read no memory. The transfers are invisible to the
// compiler's wait counting; the kernel waits for them explicitly.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m0), "v"(voff), "s"(r) : "memory");
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(m0), "v"(voff), "s"(r) : "memory");
}

__device__ int block_exclusive_scan(int v, int* tmp) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) tmp[wid] = incl;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wid; ++w) off += tmp[w];
  __syncthreads();
  return off + incl - v;
}

// Where one work item sits: rows [r0, r0 + rows) of expert e, column
// blocks [cb0, cb0 + ncb).
struct GemmTile {
  int e, r0, rows, nblk, cb0, ncb;
};

// One work item's transfer sources. With live false every offset is kOob,
// which is how an absent item (or a step past the last) is "loaded".
struct GemmSrc {
  __amdgpu_buffer_rsrc_t wr, xr;
  __amdgpu_buffer_rsrc_t sr;   // the wave's scale source: the weight scales (waves 2-5)
                               // or the rows' activation scale words (the others)
  uint32_t wo[Gemm8::dma_cb];  // per-lane weight-code offsets of the wave's transferred blocks
  uint32_t xo;           // per-lane activation offset of this wave's first row block
  uint32_t so;           // per-lane scale offset at k-step 0
  uint32_t sstep;        // its advance per k-step (per 4 k-steps for group-128 words)
};

// The fused GEMM1 epilogue (ACT): the weights are packed with the gate and
// up column blocks of each 128-column slice of h interleaved (tile nt holds
// gate blocks 8nt..8nt+7 and the matching up blocks), so each group q of 4
// packed column blocks holds gate blocks 2q, 2q+1 and their up blocks. The
// epilogue rounds both to bf16 (what GEMM1 would store), forms h =
// SiLU(g) * u and quantises one 32-column group per row exactly as
// moe_act_quant_liverows does with those bf16 inputs, and writes hq / hs.
struct GemmActOut {
  uint8_t* hq;       // [M_cap, I] E4M3
  int32_t* hs;       // [I/128, M_cap] packed UE8M0 words
  int I;
  float L;           // clamp limit (> 0: clamp)
};

static_assert(kGemmBN == 256, "the fused epilogue pairs 2 gate and 2 up blocks per group of 4");

// With half > 0 (the gate/up form of w13, half = I/16 gate column blocks)
// packed column block p takes source block src_cb(p): in each group of 16
// (one 256-column tile), position 4q + k holds gate block 8nt + 2q + k for
// k < 2 and the matching up block half + 8nt + 2q + (k - 2) for k >= 2.
__device__ __forceinline__ int src_cb(int p, int half) {
  if (half == 0) return p;
  const int nt = p >> 4, l = p & 15, q = l >> 2, k = l & 3;
  return (k < 2 ? 0 : half) + 8 * nt + 2 * q + (k & 1);
}

// The block's prologue. s_pre[e] holds, in its low
// 16 bits, the full 128-row chunks before expert e (the host caps
// M_cap / 128 < 2^16), and in its high 16 bits the rank of e's partial chunk
// (1-8 row blocks) among all partial chunks, by row blocks descending, ties
// by expert (0xFFFF: none); s_pre[E_local] is the number of full chunks F.
// Every load goes out before the first wait: this thread's experts'
// endpoints, then (ACT) its share of the compact sigmoid table, which
// reaches s_sig only after the scan has used the endpoints. Returns F and
// the number of partial chunks P, uniform over the block.
template <int THREADS, bool ACT>
__device__ __forceinline__ void gemm_prologue(const int32_t* __restrict__ expert_ends, int E_local,
                                              int A, int M_cap, int slab, int* s_pre,
                                              int* s_tmp, float* s_sig, int& F_out, int& P_out) {
  const int tid = threadIdx.x;
  constexpr int kEPT = kGemmMaxE / THREADS;   // experts per thread
  int endv[kEPT], prevv[kEPT];
#pragma unroll
  for (int j = 0; j < kEPT; ++j) {
    const int e = min(tid * kEPT + j, max(E_local - 1, 0));
    endv[j] = expert_ends[e];
    prevv[j] = expert_ends[max(e - 1, 0)];
  }
  constexpr int kSigN = ACT ? kSigRows * 128 : 1;
  constexpr int kSigPer = (kSigN + THREADS - 1) / THREADS;
  float sigv[kSigPer];
  if constexpr (ACT) {
    const float* tab = reinterpret_cast<const float*>(gemm_act::g_sigmoid_table);
#pragma unroll
    for (int j = 0; j < kSigPer; ++j) sigv[j] = tab[sigmoid_compact_source(min(tid + j * THREADS, kSigN - 1))];
  }
  int fcnt[kEPT], pblk[kEPT];
  int local_sum = 0;
#pragma unroll
  for (int j = 0; j < kEPT; ++j) {
    // expert e's live rows, as layout_range takes them from the endpoints
    // (computed for every thread, kept for e < E_local: no branch between
    // the loads and their use)
    const int e = tid * kEPT + j;
    int live_rows;
    if (slab > 0) {
      live_rows = min(max(endv[j], 0), slab);
    } else {
      const int prev = e == 0 ? 0 : min(max(prevv[j], 0), M_cap);
      const int st = min(align_up_dev(prev, A), M_cap);
      live_rows = min(max(endv[j], st), M_cap) - st;
    }
    live_rows = e < E_local ? live_rows : 0;
    fcnt[j] = live_rows / kGemmBM;
    pblk[j] = (live_rows % kGemmBM + 15) >> 4;
    local_sum += fcnt[j];
  }
  int run = block_exclusive_scan(local_sum, s_tmp);
#pragma unroll
  for (int j = 0; j < kEPT; ++j) {
    const int e = tid * kEPT + j;
    if (e < E_local) s_pre[e] = run | (pblk[j] << 16);
    run += fcnt[j];
  }
  if (tid == THREADS - 1) s_pre[E_local] = run;
  __syncthreads();
  // rank of each partial chunk (every thread walks all experts in step, so
  // each read is one broadcast); P counts the partial chunks
  int prank[kEPT];
#pragma unroll
  for (int j = 0; j < kEPT; ++j) prank[j] = 0;
  int P = 0;
  for (int e2 = 0; e2 < E_local; ++e2) {
    const int v2 = s_pre[e2] >> 16;
    P += v2 > 0;
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
      const int e = tid * kEPT + j;
      prank[j] += (v2 > pblk[j]) || (v2 == pblk[j] && e2 < e);
    }
  }
  __syncthreads();                       // every read of the row-block counts is done
#pragma unroll
  for (int j = 0; j < kEPT; ++j) {
    const int e = tid * kEPT + j;
    if (e < E_local) s_pre[e] = (s_pre[e] & 0xFFFF) | ((pblk[j] > 0 ? prank[j] : 0xFFFF) << 16);
  }
  if constexpr (ACT) {
    // published by the barrier below
#pragma unroll
    for (int j = 0; j < kSigPer; ++j)
      if (tid + j * THREADS < kSigN) s_sig[tid + j * THREADS] = sigv[j];
  }
  __syncthreads();
  // values the whole block agrees on are made scalar (readfirstlane), so
  // the buffer resources built from them stay in SGPRs
  F_out = __builtin_amdgcn_readfirstlane(s_pre[E_local]);
  P_out = __builtin_amdgcn_readfirstlane(P);
}

// The schedule. Chunks are ranked by cost: the full ones first (expert
// order), then the partial ones by row blocks descending. The full chunks
// are cut into 8 contiguous runs, one per XCD, so the chunks of an expert
// with several share its weights in one L2 where they can; the partial
// chunks are dealt in snake order (the j-th partial of XCD x is partial
// 8j + x for even j, 8j + 7 - x for odd j). Every chunk goes with all its
// NT n-tiles, so the items of a chunk share its activations in that XCD's
// L2. An XCD lists its items chunk-major (costliest first), n-tile-minor,
// and its blocks take them in snake order over rounds of nslot items, so a
// block that got a costly item in one round gets a cheap one in the next.
// (Block b runs on XCD b % 8; the grid is a multiple of 8.)
struct GemmSchedule {
  const int* s_pre;
  int E_local, A, M_cap, slab, NT, NB, F, P;
  int xcd, slot, nslot, f0, nf, nitems;

  __device__ __forceinline__ void init(const int* pre, int E, int A_, int Mc, int sl, int nt, int nb,
                                       int F_, int P_) {
    s_pre = pre; E_local = E; A = A_; M_cap = Mc; slab = sl; NT = nt; NB = nb; F = F_; P = P_;
    xcd = blockIdx.x & 7;
    slot = blockIdx.x >> 3;
    nslot = gridDim.x >> 3;
    f0 = (int)(((long long)F * xcd) >> 3);                  // this XCD's full chunks:
    nf = (int)(((long long)F * (xcd + 1)) >> 3) - f0;       // ranks [f0, f0 + nf)
    const int kr = P >> 3, rm = P & 7;     // full rounds of partial chunks, remainder
    const int nx = nf + kr + (((kr & 1) ? 7 - xcd : xcd) < rm);   // chunks of this XCD
    nitems = nx * NT;
  }
  // the block's k-th item (an index into the XCD's list), or -1 past its last
  __device__ __forceinline__ int item_at(int k) const {
    const int u = nslot * k + ((k & 1) ? nslot - 1 - slot : slot);
    return u < nitems ? u : -1;
  }
  __device__ __forceinline__ void locate(int item, GemmTile& T,
                                         const int32_t* __restrict__ expert_ends) const {
    const int lane = threadIdx.x & 63;
    const int kq = item / NT;
    const int nt = item - kq * NT;
    const int jp = kq - nf;                                  // partial index, if >= 0
    const int r = jp < 0 ? f0 + kq : F + 8 * jp + ((jp & 1) ? 7 - xcd : xcd);   // chunk rank
    int e, c;
    if (r < F) {
      // full chunk r: the last expert whose full-chunk prefix is <= r
      int lo = 0, hi = E_local - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const int pm = __builtin_amdgcn_readfirstlane(s_pre[mid]) & 0xFFFF;
        if (pm <= r) lo = mid; else hi = mid - 1;
      }
      e = lo;
      c = r - (__builtin_amdgcn_readfirstlane(s_pre[e]) & 0xFFFF);
    } else {
      // partial chunk of rank r - F: the expert holding that rank
      const int want = r - F;
      e = 0;
      for (int e0 = 0; e0 < E_local; e0 += 64) {
        const int ee = e0 + lane;
        const uint64_t hit = __ballot(ee < E_local && (s_pre[min(ee, E_local - 1)] >> 16) == want);
        if (hit) {
          e = e0 + __ffsll((unsigned long long)hit) - 1;
          break;
        }
      }
      e = __builtin_amdgcn_readfirstlane(e);
      c = (__builtin_amdgcn_readfirstlane(s_pre[e + 1]) & 0xFFFF) -
          (__builtin_amdgcn_readfirstlane(s_pre[e]) & 0xFFFF);        // e's full chunks
    }
    // expert e's live rows, as layout_range takes them; both endpoint
    // loads are issued before either is used (one round trip)
    const int endv_e = expert_ends[e];
    const int prevv_e = expert_ends[max(e - 1, 0)];
    int start, end;
    if (slab > 0) {
      start = e * slab;
      end = start + min(max(endv_e, 0), slab);
    } else {
      const int prev = e == 0 ? 0 : min(max(prevv_e, 0), M_cap);
      start = min(align_up_dev(prev, A), M_cap);
      end = min(max(endv_e, start), M_cap);
    }
    start = __builtin_amdgcn_readfirstlane(start);
    end = __builtin_amdgcn_readfirstlane(end);
    T.e = e;
    T.r0 = start + c * kGemmBM;
    T.rows = min(kGemmBM, end - T.r0);                   // >= 1
    T.nblk = (T.rows + 15) >> 4;
    T.cb0 = nt * (kGemmBN / 16);
    T.ncb = min(kGemmBN / 16, NB - T.cb0);
  }
};

// The fused activation of one row block and one 32-column h group: gate
// column blocks g0, g1 and their up blocks u0, u1 (lane holds columns
// 16c + 4(lane/16) .. +3 of each block). h[c][j] receives the lane's 8
// values of h and the return value their group's amax (the 4 lanes l16 + 16
// g' of a row agree on it). Runs on every lane of the wave (the amax
// reduction and the small-sigma ballot are wave-wide).
__device__ __forceinline__ float act_h_group(const v4f& g0, const v4f& g1, const v4f& u0,
                                             const v4f& u1, const float* s_sig,
                                             const GemmActOut& act, float (&h)[2][4]) {
  // gate and up rounded to bf16 (RNE, NaN -> the quiet NaN 0x7FC0: the
  // values moe_grouped_gemm1 stores), two per conversion
  float gv[8], uv[8];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const v4f g4 = c == 0 ? g0 : g1, u4 = c == 0 ? u0 : u1;
    const float ga[4] = {g4.x, g4.y, g4.z, g4.w};
    const float ua[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w = bf16x2_rne_bits(ga[k], ua[k]);
      gv[4 * c + k] = ga[k] != ga[k] ? __uint_as_float(0x7FC00000u) : __uint_as_float(w << 16);
      uv[4 * c + k] = ua[k] != ua[k] ? __uint_as_float(0x7FC00000u) : __uint_as_float(w & 0xFFFF0000u);
    }
  }
  if (act.L > 0.f) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      gv[k] = fminf(gv[k], act.L);
      uv[k] = fminf(fmaxf(uv[k], -act.L), act.L);
    }
  }
  float sig[8];
  bool small = false;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    sig[k] = sigmoid_lookup_compact_fast(s_sig, gv[k]);
    small |= sigmoid_is_small(gv[k]);
  }
  if (__builtin_amdgcn_ballot_w64(small)) {                 // rare: |g| < 2^-15
#pragma unroll
    for (int k = 0; k < 8; ++k) sig[k] = sigmoid_small_fix(gv[k], sig[k]);
  }
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float sg = gv[k] * sig[k];
    h[k >> 2][k & 3] = sg * uv[k];
    amax = fmaxf(amax, fabsf(h[k >> 2][k & 3]));
  }
  // the 32-column group of this row spans lanes l16 + 16 g'
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  return amax;
}

// The E4M3 codes of a lane's 8 h values of tile row mr with the UE8M0 byte
// bsc, at h columns 128 nt + 32 q + 16 c + 4(lane/16) .. +3 (c = 0, 1).
__device__ __forceinline__ void act_store_codes(const float (&h)[2][4], uint32_t bsc,
                                                const GemmActOut& act, const GemmTile& T, int mr,
                                                int nt, int q) {
  const int g = (threadIdx.x & 63) >> 4;
  const float inv = e8m0_reciprocal(bsc);
  if (mr < T.rows) {
    const size_t row = (size_t)(T.r0 + mr);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t w = 0;
      w = cvt_e4m3x2<false>(h[c][0] * inv, h[c][1] * inv, w);
      w = cvt_e4m3x2<true>(h[c][2] * inv, h[c][3] * inv, w);
      *reinterpret_cast<uint32_t*>(act.hq + row * act.I + 128 * nt + 32 * q + 16 * c + 4 * g) = w;
    }
  }
}

// The group-32 fused activation of one row block and one h group (group q
// of slice nt): h, its own 32-column scale byte, the codes, and byte q of
// the row's scale word of slice nt (group 4 nt + q).
__device__ __forceinline__ void act_epilogue_group(const v4f& g0, const v4f& g1, const v4f& u0,
                                                   const v4f& u1, const float* s_sig,
                                                   const GemmActOut& act, const GemmTile& T,
                                                   int mr, int nt, int q, int slab, int ss) {
  const int g = (threadIdx.x & 63) >> 4;
  float h[2][4];
  const uint32_t bsc = ue8m0_byte_of_amax(act_h_group(g0, g1, u0, u1, s_sig, act, h));
  act_store_codes(h, bsc, act, T, mr, nt, q);
  if (mr < T.rows && g == 0) {
    const size_t row = (size_t)(T.r0 + mr);
    const size_t hs0 = slab > 0 ? (size_t)T.e * (size_t)(act.I / 128 - 1) * (size_t)slab : 0;
    reinterpret_cast<uint8_t*>(act.hs)[(hs0 + (size_t)nt * ss + row) * 4 + q] = (uint8_t)bsc;
  }
}

// XG128: activation scales of one UE8M0 byte per 128 columns, packed four
// k-steps to a word ([ceil(K/512)][M_cap]); the byte of k-step ks is byte
// ks % 4 of word ks / 4 and serves all four 32-column blocks of the step.
// NATW: the weights in their checkpoint layout (codes [E][N][K/2], scales
// [E][N][K/32]) instead of the packed one. Each lane's 16 code bytes of a
// k-step are then the 64-byte run [64 ks + 16 (l/16), +16) of row
// 16 cb + l%16 (the packed chunk is exactly these bytes, so the LDS stage is
// the same), and the tile's scales of a k-step are one dword per weight row
// (its 4 groups), moved by waves 2-5 and gathered into the MFMA's scale word
// by 4 byte reads. With ACT the gate/up interleaving of the packed form is
// an address mapping (src_cb).
template <bool ACT, bool XG128, bool NATW>
__global__ __launch_bounds__(Gemm8::threads, 1) void grouped_mx_gemm_kernel(
    const uint8_t* __restrict__ X, const int32_t* __restrict__ Xs,
    const int32_t* __restrict__ expert_ends, int E_local, int A, int M_cap, int slab, int K, int N,
    const uint8_t* __restrict__ Wp, const uint8_t* __restrict__ Sp, uint16_t* __restrict__ out,
    GemmActOut act) {
  using L = Gemm8;
  constexpr int kGemmCB = L::CB, kGemmCG = L::CG, kDmaCB = L::dma_cb, kDmaXR = L::dma_xr;
  constexpr int kDmaOps = kDmaCB + 2 * kDmaXR;
  __shared__ GemmStage stage[kGemmStages];
  __shared__ int s_pre[kGemmMaxE + 1];
  __shared__ int s_tmp[L::waves];
  // the fused epilogue's sigmoid values (the compact subset of the table)
  __shared__ __attribute__((aligned(16))) float s_sig[ACT ? kSigRows * 128 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int rg = wid / kGemmCG;          // MFMA rows: row blocks [MB rg, MB rg + MB)
  const int cg = wid % kGemmCG;          // MFMA columns: column blocks [CB cg, CB cg + CB)
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int KS = K / 128;                // k-steps
  const int NB = N / 16;                 // column blocks
  // activation scale words per row, and the distance between a row's
  // consecutive words: the whole buffer's rows (aligned layout) or one
  // expert's slab (masked layout, where expert e's words start at
  // e * XW * slab)
  const int XW = XG128 ? (KS + 3) / 4 : KS;
  const int ss = slab > 0 ? slab : M_cap;
  const int NT = (N + kGemmBN - 1) / kGemmBN;

  int F, P;
  gemm_prologue<L::threads, ACT>(expert_ends, E_local, A, M_cap, slab, s_pre, s_tmp, s_sig, F, P);
  if (F + P == 0) return;                // no live rows (uniform over the block)
  GemmSchedule sch;
  sch.init(s_pre, E_local, A, M_cap, slab, NT, NB, F, P);

  // weight column block of packed position p (the gate/up interleave of the
  // fused form; identity otherwise)
  const int half = ACT ? act.I / 16 : 0;
  // waves 2-5 move the tile's weight scales, the others the rows' scale words
  const bool wsw = wid >= 2 && wid < 6;
  const uint32_t s_lds = wsw ? (uint32_t)(kOffWs + (wid - 2) * 256) : (uint32_t)(kOffXs + (wid & 1) * 256);
  auto sources = [&](const GemmTile& T, bool live) {
    GemmSrc q;
    if constexpr (NATW) {
      q.wr = make_rsrc(Wp + (size_t)T.e * N * (K / 2), (uint32_t)N * (uint32_t)(K / 2));
    } else {
      q.wr = make_rsrc(Wp + ((size_t)T.e * NB + T.cb0) * KS * 1024, (uint32_t)(T.ncb * KS) * 1024u);
    }
    q.xr = make_rsrc(X + (size_t)T.r0 * K, (uint32_t)T.rows * (uint32_t)K);
    if (wsw) {
      q.sr = NATW ? make_rsrc(Sp + (size_t)T.e * N * (K / 32), (uint32_t)N * (uint32_t)(K / 32))
                  : make_rsrc(Sp + (size_t)T.e * KS * NB * 64, (uint32_t)(KS * NB) * 64u);
    } else {
      // scale word w of row r: [w][r] (aligned layout), [e][w][r - e slab] (slab)
      const size_t xs0 = (slab > 0 ? (size_t)T.e * (size_t)(XW - 1) * (size_t)slab : 0) + T.r0;
      q.sr = make_rsrc(Xs + xs0, (uint32_t)((XW - 1) * ss + T.rows) * 4u);
    }
#pragma unroll
    for (int c = 0; c < kDmaCB; ++c) {
      const int cb = kDmaCB * wid + c;
      if constexpr (NATW) {
        const int src = src_cb(T.cb0 + cb, half);
        q.wo[c] = (live && cb < T.ncb) ? (uint32_t)(16 * src + l16) * (uint32_t)(K / 2) + 16 * g : kOob;
      } else {
        q.wo[c] = (live && cb < T.ncb) ? (uint32_t)(cb * KS) * 1024u + lane * 16 : kOob;
      }
    }
    q.xo = (live && 16 * kDmaXR * wid < T.rows)
               ? (uint32_t)(16 * kDmaXR * wid + l16) * (uint32_t)K + 16 * g : kOob;
    if (!wsw) {
      // rows 64 (wid & 1) + lane (waves 6, 7 repeat waves 0, 1)
      q.so = (live && 64 * (wid & 1) < T.rows) ? (uint32_t)(64 * (wid & 1) + lane) * 4u : kOob;
      q.sstep = (uint32_t)ss * 4u;
    } else if constexpr (NATW) {
      // tile weight row n = 64 (wid - 2) + lane, its 4 groups of the step
      const int n = 64 * (wid - 2) + lane, cbt = n >> 4;
      q.so = (live && cbt < T.ncb)
                 ? (uint32_t)(16 * src_cb(T.cb0 + cbt, half) + (n & 15)) * (uint32_t)(K / 32)
                 : kOob;
      q.sstep = 4u;
    } else {
      // group wid - 2 of the tile's 4 (256 bytes of one contiguous 1 KB block)
      q.so = live ? (uint32_t)((T.cb0 >> 2) * 256 + (wid - 2) * 256 + lane * 4) : kOob;
      q.sstep = (uint32_t)(64 * NB);
    }
    return q;
  };

  const uint32_t lds0 = (uint32_t)(uintptr_t)&stage[0];
  // transfers of k-step st of a source into ring stage sg: per wave its 2
  // weight blocks, the 2 halves of its activation row block and one dword
  // per lane of scales (waves 2-5: a quarter of the tile's weight scales;
  // waves 0, 1: the scale words of rows 64 w .. + 63, repeated by 6, 7)
  auto issue_op = [&](const GemmSrc& q, int st, int sg, auto kk) {
    constexpr int k = decltype(kk)::value;
    const uint32_t base = lds0 + (uint32_t)sg * (uint32_t)sizeof(GemmStage);
    if constexpr (k < kDmaCB) {
      dma16(q.wr, q.wo[k] + (uint32_t)st * (NATW ? 64u : 1024u), base + kOffW + (kDmaCB * wid + k) * 1024);
    } else if constexpr (k < kDmaOps) {
      constexpr int r = (k - kDmaCB) / 2, h = (k - kDmaCB) % 2;
      dma16(q.xr, q.xo + (uint32_t)(16 * r) * (uint32_t)K + (uint32_t)st * 128u + 64 * h,
            base + (kDmaXR * wid + r) * 2048 + h * 1024);
    } else {
      // one dword per lane on every wave (no per-wave branch in the step)
      static_assert(kGemmBN / 16 == 16, "4 waves of 256 bytes cover the tile's weight scales");
      const int sk = (XG128 && !wsw) ? st >> 2 : st;
      dma4(q.sr, q.so + (uint32_t)sk * q.sstep, base + s_lds);
    }
  };
  auto issue = [&](const GemmSrc& q, int st, int sg) {
    issue_op(q, st, sg, std::integral_constant<int, 0>{});
    issue_op(q, st, sg, std::integral_constant<int, 1>{});
    issue_op(q, st, sg, std::integral_constant<int, 2>{});
    issue_op(q, st, sg, std::integral_constant<int, 3>{});
    issue_op(q, st, sg, std::integral_constant<int, 4>{});
    static_assert(kDmaOps + 1 == 5 && L::ops == 5, "issue covers 5 transfers");
  };
  // waits until this wave's transfers of the oldest stage in flight have
  // landed: kGemmStages - 2 stages (kDmaOps + 1 transfers each) were issued
  // after it
  constexpr int kWaitA = (kGemmStages - 2) * (kDmaOps + 1);
  static_assert(kWaitA < 64, "vmcnt field");
  static_assert(L::waves == 8, "waves 0, 1, 6, 7 move scale words, waves 2-5 weight scales");
  auto wait_stage = [&]() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kWaitA) : "memory"); };

  int kc = 0;                            // the block's current item (k-th)
  int item = sch.item_at(0);
  bool valid = item >= 0;
  GemmTile T{0, 0, 1, 1, 0, 0};
  if (valid) sch.locate(item, T, expert_ends);
  // the transfer walker: item kp, step pst, its sources; it runs 3 steps
  // ahead of the compute and steps into the block's next item (or past the
  // last, into sources that read nothing) at an item's end
  int kp = 0, pst = 0;
  GemmSrc ps = sources(T, valid);
  auto advance = [&]() {
    if (++pst == KS) {
      pst = 0;
      const int u = sch.item_at(++kp);
      GemmTile U = T;
      if (u >= 0) sch.locate(u, U, expert_ends);
      ps = sources(U, u >= 0);
    }
  };
  int gs = 0;                            // running k-step count; ring stage gs % 4
  if (valid) {
    for (int s = 0; s < kGemmStages - 1; ++s) {
      issue(ps, pst, s);
      advance();
    }
  }
  while (valid) {
    // this wave's live row blocks among its kGemmMB
    const int mlive = min(max(T.nblk - kGemmMB * rg, 0), kGemmMB);

    v4f acc[kGemmCB][kGemmMB];
#pragma unroll
    for (int c = 0; c < kGemmCB; ++c)
#pragma unroll
      for (int i = 0; i < kGemmMB; ++i) acc[c][i] = v4f{0.f, 0.f, 0.f, 0.f};

    // The operands of one k-step in registers: the wave's 4 weight
    // fragments and their scale word, the scale words of its row blocks, and
    // the activation fragments of row block i in bf[i].
    struct StepOps {
      v4i af[kGemmCB];
      int sa;
      uint32_t xw[kGemmMB];
      v8i bf[kGemmMB];
    };
    static_assert(kGemmCB == 4, "one scale word covers the wave's 4 column blocks");
    // activation fragments of row block i of the current stage; a row block
    // past the live ones is read as one broadcast word
    auto read_b = [&](StepOps& o, int i, auto full) {
      constexpr bool FULL = decltype(full)::value;
      const GemmStage& S = stage[gs % kGemmStages];
      const bool live = FULL || i < mlive;
      const uint8_t* xb = &S.x[0][0][0];
      const int off = live ? (kGemmMB * rg + i) * 2048 + lane * 16 : 0;
      const v4i lo4 = *reinterpret_cast<const v4i*>(xb + off);
      const v4i hi4 = *reinterpret_cast<const v4i*>(xb + off + (live ? 1024 : 0));
      o.bf[i] = v8i{lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
    };
    // the head of step gs: wait until its stage is complete for this wave,
    // then (barrier) for the block, and read its weight fragments, scale
    // words and the first two row blocks' activation fragments. The barrier
    // also retires every read of the stage that step gs refills, provided
    // each wave's reads of it have completed before the wave arrives.
    auto head = [&](StepOps& o, auto full) {
      wait_stage();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const GemmStage& S = stage[gs % kGemmStages];
#pragma unroll
      for (int c = 0; c < kGemmCB; ++c)
        o.af[c] = *reinterpret_cast<const v4i*>(&S.w[kGemmCB * cg + c][lane * 16]);
      if constexpr (NATW) {
        // byte g of tile row 16 (4 cg + c) + l16's dword, for c = 0..3
        const uint8_t* wsb = &S.ws[0][0];
        uint32_t v = 0;
#pragma unroll
        for (int c = 0; c < kGemmCB; ++c)
          v |= (uint32_t)wsb[(16 * (kGemmCB * cg + c) + l16) * 4 + g] << (8 * c);
        o.sa = (int)v;
      } else {
        o.sa = (int)*reinterpret_cast<const uint32_t*>(&S.ws[0][0] + 256 * cg + 4 * lane);
      }
#pragma unroll
      for (int i = 0; i < kGemmMB; ++i) o.xw[i] = S.xs[16 * (kGemmMB * rg + i) + l16];
      read_b(o, 0, full);
      read_b(o, 1, full);
    };

    // one k-step on operands whose head is in o. FULL (all of the wave's
    // row blocks live) runs without per-row-block branches. PIPE: the next
    // step's head is taken (into nx) before the last row block's MFMAs, so
    // the matrix cores work through the barrier; nx must not be o.
    int cur_ks = 0;                      // the item's k-step (XG128 picks the scale byte by it)
    auto step = [&](StepOps& o, StepOps& nx, auto full, auto walk, auto pipe) {
      constexpr bool FULL = decltype(full)::value;
      constexpr bool WALK = decltype(walk)::value;
      constexpr bool PIPE = decltype(pipe)::value;
      // transfers of the walker's step (3 ahead) into the stage the
      // previous step used
      const int sg = (gs + kGemmStages - 1) % kGemmStages;
      const int xk = XG128 ? (cur_ks & 3) : g;    // scale byte of the step's k-block
      auto mfmas = [&](int i) {
        if (FULL || i < mlive) {
          const int sb = (int)(o.xw[i] >> (8 * xk));
          // op_sel must be a constant: one call per column block
          auto mfma = [&](auto cc) {
            constexpr int c = decltype(cc)::value;
            acc[c][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                o.af[c].xyzwxyzw, o.bf[i], acc[c][i], 4, 0, c, o.sa, 0, sb);
          };
          mfma(std::integral_constant<int, 0>{});
          mfma(std::integral_constant<int, 1>{});
          mfma(std::integral_constant<int, 2>{});
          mfma(std::integral_constant<int, 3>{});
        }
      };
      static_assert(kGemmMB == 4 && kDmaOps + 1 == 5, "the step below spreads 5 transfers over 4 row blocks");
      // two transfers after each of the first row blocks' MFMAs, so the
      // block's transfers spread over the step instead of queueing at its
      // start (the scheduling barriers keep this order)
      read_b(o, 2, full);
      mfmas(0);
      __builtin_amdgcn_sched_barrier(0);
      issue_op(ps, pst, sg, std::integral_constant<int, 0>{});
      issue_op(ps, pst, sg, std::integral_constant<int, 1>{});
      __builtin_amdgcn_sched_barrier(0);
      read_b(o, 3, full);
      mfmas(1);
      __builtin_amdgcn_sched_barrier(0);
      issue_op(ps, pst, sg, std::integral_constant<int, 2>{});
      issue_op(ps, pst, sg, std::integral_constant<int, 3>{});
      __builtin_amdgcn_sched_barrier(0);
      mfmas(2);
      __builtin_amdgcn_sched_barrier(0);
      issue_op(ps, pst, sg, std::integral_constant<int, 4>{});
      __builtin_amdgcn_sched_barrier(0);
      // the walker enters the next item only in an item's last 4 steps
      // (it runs 3 ahead); before those the step body has no branch
      if constexpr (WALK) advance(); else ++pst;
      ++gs;
      if constexpr (PIPE) {
        // this wave's reads of the stage are complete before it arrives
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        head(nx, full);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfmas(3);
      __builtin_amdgcn_sched_barrier(0);
    };
    const int ks_plain = KS - 4;         // steps [0, KS - 4): no item change in the walker
    auto run_item = [&](auto full) {
      StepOps o[2];
      head(o[0], full);
      int ks = 0;
      for (; ks + 2 <= ks_plain; ks += 2) {
        cur_ks = ks;
        step(o[0], o[1], full, std::false_type{}, std::true_type{});
        cur_ks = ks + 1;
        step(o[1], o[0], full, std::false_type{}, std::true_type{});
      }
      if (ks < ks_plain) {
        cur_ks = ks;
        step(o[0], o[1], full, std::false_type{}, std::true_type{});
        o[0] = o[1];
        ++ks;
      }
      for (; ks < KS; ++ks) {
        cur_ks = ks;
        step(o[0], o[1], full, std::true_type{}, std::false_type{});
        if (ks + 1 < KS) head(o[0], full);
      }
    };
    if (mlive == kGemmMB) run_item(std::true_type{});
    else run_item(std::false_type{});

    if constexpr (!ACT) {
      // epilogue: lane holds columns 16cb + 4g .. +3 of row r0 + 16mb + l16
#pragma unroll
      for (int c = 0; c < kGemmCB; ++c) {
        const int cb = kGemmCB * cg + c;
        if (cb >= T.ncb) continue;
        const int n = (T.cb0 + cb) * 16 + 4 * g;
#pragma unroll
        for (int i = 0; i < kGemmMB; ++i) {
          const int mr = 16 * (kGemmMB * rg + i) + l16;
          if (i >= mlive || mr >= T.rows) continue;
          const v4f v = acc[c][i];
          const uint2 o = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
          *reinterpret_cast<uint2*>(out + (size_t)(T.r0 + mr) * N + n) = o;
        }
      }
    } else if constexpr (!XG128) {
      // fused activation: the wave's 4 column blocks are group cg of the
      // 128-column slice nt = cb0 / 16
      const int nt = T.cb0 >> 4;
#pragma unroll
      for (int i = 0; i < kGemmMB; ++i) {
        if (i >= mlive) continue;                            // wave-uniform
        act_epilogue_group(acc[0][i], acc[1][i], acc[2][i], acc[3][i], s_sig, act, T,
                           16 * (kGemmMB * rg + i) + l16, nt, cg, slab, ss);
      }
    } else {
      // fused activation, group-128 output: slice nt's 128 h columns are
      // one group, spread over the 4 column-group waves of a row group; each
      // wave's 32-column amax per row goes through LDS. The exchange uses
      // the stage the item's last step read: the next transfer into it is
      // issued after the next step's barrier. The first barrier lets every
      // wave finish that last step's reads of it.
      const int nt = T.cb0 >> 4;
      float* xa = reinterpret_cast<float*>(&stage[(gs + kGemmStages - 1) % kGemmStages]);
      float hv[kGemmMB][2][4];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kGemmMB; ++i) {
        if (i >= mlive) continue;                            // wave-uniform
        const float amax = act_h_group(acc[0][i], acc[1][i], acc[2][i], acc[3][i], s_sig, act, hv[i]);
        if (g == 0) xa[((kGemmMB * rg + i) * 16 + l16) * 4 + cg] = amax;
      }
      __syncthreads();
      const int NTh = act.I >> 7;          // 128-column groups of h
#pragma unroll
      for (int i = 0; i < kGemmMB; ++i) {
        if (i >= mlive) continue;
        const int mr = 16 * (kGemmMB * rg + i) + l16;
        const v4f a4 = *reinterpret_cast<const v4f*>(&xa[((kGemmMB * rg + i) * 16 + l16) * 4]);
        const float amax = fmaxf(fmaxf(a4.x, a4.y), fmaxf(a4.z, a4.w));
        const uint32_t bsc = ue8m0_byte_of_amax(amax);
        act_store_codes(hv[i], bsc, act, T, mr, nt, cg);
        // byte nt % 4 of the row's word nt / 4; the bytes of groups past I
        // in the last word are 0
        if (cg == 0 && g == 0 && mr < T.rows) {
          uint8_t* hb = reinterpret_cast<uint8_t*>(act.hs) + ((size_t)(nt >> 2) * ss + T.r0 + mr) * 4;
          hb[nt & 3] = (uint8_t)bsc;
          if (nt == NTh - 1)
            for (int z = (nt & 3) + 1; z < 4; ++z) hb[z] = 0;
        }
      }
    }
    // (the stores above share the counter with the transfers; they may
    // complete before older transfers, but the transfers complete in order,
    // so counting transfers alone in wait_stage still waits for the stage)
    item = sch.item_at(++kc);
    valid = item >= 0;
    if (valid) sch.locate(item, T, expert_ends);
  }
  // every transfer this block issued has landed before its LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Load-time weight preparation (bit-exact data movement):
//   codes  w [E][N][K/2] -> wp [E][N/16][K/128][64 lanes][16 B]
//          lane l of chunk (e, cb, ks) = bytes [64ks + 16(l/16), +16) of row 16cb + l%16
//   scales s [E][N][K/32] -> sp [E][K/128][N/64][64 lanes][4 B]
//          byte b of lane l's word of group q in (e, ks) = group 4ks + l/16 of
//          row 16(4q + b) + l%16
// One wave per 1 KB code chunk; one thread per scale byte.
//
__global__ __launch_bounds__(256) void pack_mx_codes_kernel(const uint8_t* __restrict__ w, int N,
                                                            int K, int half, uint8_t* __restrict__ wp) {
  const int KS = K / 128;
  const size_t per_e = (size_t)(N / 16) * KS;
  const size_t chunk = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (chunk >= per_e) return;
  const int e = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int cb = (int)(chunk / KS);
  const int ks = (int)(chunk - (size_t)cb * KS);
  const size_t row = (size_t)e * N + 16 * src_cb(cb, half) + (lane & 15);
  const uint4 v =
      *reinterpret_cast<const uint4*>(w + row * (size_t)(K / 2) + 64 * ks + 16 * (lane >> 4));
  *reinterpret_cast<uint4*>(wp + ((size_t)e * per_e + chunk) * 1024 + lane * 16) = v;
}

__global__ __launch_bounds__(256) void pack_mx_scales_kernel(const uint8_t* __restrict__ s, int N,
                                                             int K, int half, uint8_t* __restrict__ sp) {
  const int NB = N / 16;
  const size_t per_e = (size_t)(K / 128) * 64 * NB;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= per_e) return;
  const int e = blockIdx.y;
  // idx = ((ks * NB/4 + q) * 64 + l) * 4 + b: byte b of lane l's word of
  // column-block group q (block 4q + b) in k-step ks
  const int b = (int)(idx & 3);
  const int l = (int)((idx >> 2) & 63);
  const size_t gq = idx >> 8;                    // ks * NB/4 + q
  const int ks = (int)(gq / (NB / 4));
  const int cb = 4 * (int)(gq - (size_t)ks * (NB / 4)) + b;
  sp[(size_t)e * per_e + idx] =
      s[((size_t)e * N + 16 * src_cb(cb, half) + (l & 15)) * (size_t)(K / 32) + 4 * ks + (l >> 4)];
}

// slab == 0: the aligned layout (ends = expert_ends, M_cap rows); slab =
// m_pad > 0: the masked slab layout (ends = masked_m, M_cap = E_local * m_pad)
static int launch_grouped_gemm(const uint8_t* X, const int32_t* Xs, const int32_t* ends,
                               int E_local, int A, int M_cap, int K, int N, const uint8_t* Wp,
                               const uint8_t* Sp, uint16_t* out, void* stream,
                               const GemmActOut* act = nullptr, bool xg128 = false,
                               int slab = 0, bool natw = false) {
  if (E_local < 0 || E_local > kGemmMaxE || A < 1 || M_cap < 0 || K <= 0 || N <= 0)
    return MOE_ERR_SHAPE;
  if (K % 128 != 0 || N % 128 != 0 || M_cap % 4 != 0) return MOE_ERR_ALIGN;
  // buffer ranges are 32-bit: one expert's packed weights and one 128-row
  // activation chunk must stay below 2 GiB
  if ((long long)N * K / 2 >= (1LL << 31) || (long long)kGemmBM * K >= (1LL << 31) ||
      (long long)(K / 128) * M_cap * 4 >= (1LL << 31))
    return MOE_ERR_SHAPE;
  // the in-kernel chunk scan packs full-chunk counts into 16 bits
  if (M_cap / kGemmBM >= (1 << 16)) return MOE_ERR_SHAPE;
  if (E_local == 0 || M_cap == 0) return MOE_OK;
  if (!X || !Xs || !ends || !Wp || !Sp || (!out && !act)) return MOE_ERR_NULL;
  // one resident block per CU; each walks its XCD's share of the item list
  const int NT = (N + kGemmBN - 1) / kGemmBN;
  const long long max_items = (long long)((M_cap + kGemmBM - 1) / kGemmBM + E_local) * NT;
  const int resident = 256;
  int grid = max_items < resident ? (int)max_items : resident;
  grid = (grid + 7) & ~7;
  if (natw && xg128) return MOE_ERR_UNSUPPORTED;   // natural weights with group-32 activations only
  if (act && xg128 && slab > 0) return MOE_ERR_UNSUPPORTED;   // group 128: aligned layout only
  const GemmActOut a = act ? *act : GemmActOut{nullptr, nullptr, 0, 0.f};
  if (act) {
    auto kernel = natw    ? grouped_mx_gemm_kernel<true, false, true>
                  : xg128 ? grouped_mx_gemm_kernel<true, true, false>
                          : grouped_mx_gemm_kernel<true, false, false>;
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(Gemm8::threads), 0, (hipStream_t)stream, X, Xs,
                       ends, E_local, A, M_cap, slab, K, N, Wp, Sp, out, a);
  } else {
    auto kernel = natw ? grouped_mx_gemm_kernel<false, false, true>
                  : xg128 ? grouped_mx_gemm_kernel<false, true, false>
                          : grouped_mx_gemm_kernel<false, false, false>;
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(Gemm8::threads), 0, (hipStream_t)stream, X, Xs,
                       ends, E_local, A, M_cap, slab, K, N, Wp, Sp, out, a);
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

static int pack_mx(const uint8_t* w, const uint8_t* w_scale, int E, int N, int K, int half,
                   uint8_t* w_packed, uint8_t* w_scale_packed, void* stream) {
  if (E < 0 || N < 0 || K <= 0 || E > 65535) return MOE_ERR_SHAPE;
  if (K % 128 != 0 || N % 64 != 0) return MOE_ERR_ALIGN;
  if (E == 0 || N == 0) return MOE_OK;
  if (!w || !w_scale || !w_packed || !w_scale_packed) return MOE_ERR_NULL;
  const size_t chunks = (size_t)(N / 16) * (K / 128);
  const size_t scale_bytes = (size_t)N * (K / 32);
  if ((chunks + 3) / 4 > 0x7fffffffu || (scale_bytes + 255) / 256 > 0x7fffffffu) return MOE_ERR_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(pack_mx_codes_kernel, dim3((unsigned)((chunks + 3) / 4), (unsigned)E),
                     dim3(256), 0, st, w, N, K, half, w_packed);
  MOE_CHECK_LAUNCH();
  hipLaunchKernelGGL(pack_mx_scales_kernel, dim3((unsigned)((scale_bytes + 255) / 256), (unsigned)E),
                     dim3(256), 0, st, w_scale, N, K, half, w_scale_packed);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

}  // namespace moe

extern "C" int moe_pack_mx_weights(const uint8_t* w, const uint8_t* w_scale, int E, int N, int K,
                                   uint8_t* w_packed, uint8_t* w_scale_packed, void* stream) {
  return moe::pack_mx(w, w_scale, E, N, K, 0, w_packed, w_scale_packed, stream);
}

extern "C" int moe_pack_mx_weights_gateup(const uint8_t* w13, const uint8_t* w13_scale, int E,
                                          int I, int H, uint8_t* w_packed,
                                          uint8_t* w_scale_packed, void* stream) {
  if (I <= 0 || I % 128 != 0) return MOE_ERR_ALIGN;
  return moe::pack_mx(w13, w13_scale, E, 2 * I, H, I / 16, w_packed, w_scale_packed, stream);
}

extern "C" int moe_grouped_gemm1(const uint8_t* xq, const int32_t* xs, const int32_t* expert_ends,
                                 int E_local, int A, int M_cap, int H, int I,
                                 const uint8_t* w13_packed, const uint8_t* w13_scale_packed,
                                 uint16_t* gateup, void* stream) {
  if (I <= 0 || I % 64 != 0) return MOE_ERR_ALIGN;
  return moe::launch_grouped_gemm(xq, xs, expert_ends, E_local, A, M_cap, H, 2 * I, w13_packed,
                                  w13_scale_packed, gateup, stream);
}

extern "C" int moe_grouped_gemm2(const uint8_t* hq, const int32_t* hs, const int32_t* expert_ends,
                                 int E_local, int A, int M_cap, int I, int H,
                                 const uint8_t* w2_packed, const uint8_t* w2_scale_packed,
                                 uint16_t* down, void* stream) {
  return moe::launch_grouped_gemm(hq, hs, expert_ends, E_local, A, M_cap, I, H, w2_packed,
                                  w2_scale_packed, down, stream);
}

extern "C" int moe_grouped_gemm1_g128(const uint8_t* xq, const int32_t* xs,
                                      const int32_t* expert_ends, int E_local, int A, int M_cap,
                                      int H, int I, const uint8_t* w13_packed,
                                      const uint8_t* w13_scale_packed, uint16_t* gateup,
                                      void* stream) {
  if (I <= 0 || I % 64 != 0) return MOE_ERR_ALIGN;
  return moe::launch_grouped_gemm(xq, xs, expert_ends, E_local, A, M_cap, H, 2 * I, w13_packed,
                                  w13_scale_packed, gateup, stream, nullptr, true);
}

extern "C" int moe_grouped_gemm2_g128(const uint8_t* hq, const int32_t* hs,
                                      const int32_t* expert_ends, int E_local, int A, int M_cap,
                                      int I, int H, const uint8_t* w2_packed,
                                      const uint8_t* w2_scale_packed, uint16_t* down,
                                      void* stream) {
  return moe::launch_grouped_gemm(hq, hs, expert_ends, E_local, A, M_cap, I, H, w2_packed,
                                  w2_scale_packed, down, stream, nullptr, true);
}

namespace {
// The clamp rule of moe_act_quant_liverows: L <= 0 or +inf: none; a finite
// L > 0 must be exactly representable in bf16; NaN is rejected.
int fused_clamp(float clamp_limit, float& L) {
  L = 0.f;
  if (clamp_limit > 0.f && clamp_limit < __builtin_inff()) {
    uint32_t bits;
    std::memcpy(&bits, &clamp_limit, 4);
    if (bits & 0xFFFFu) return MOE_ERR_UNSUPPORTED;
    L = clamp_limit;
  } else if (!(clamp_limit <= 0.f) && !(clamp_limit == __builtin_inff())) {
    return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

// Masked slab sizes: m_pad a multiple of 4 (the scale words' MN direction),
// E_local * m_pad rows addressable with 32-bit row indices.
int masked_rows(int E_local, int m_pad, int& M_cap) {
  if (E_local < 0 || m_pad < 0) return MOE_ERR_SHAPE;
  if (m_pad % 4 != 0) return MOE_ERR_ALIGN;
  if ((long long)E_local * m_pad >= (1LL << 31)) return MOE_ERR_SHAPE;
  M_cap = E_local * m_pad;
  return MOE_OK;
}
}  // namespace

extern "C" int moe_grouped_gemm1_act_quant(const uint8_t* xq, const int32_t* xs,
                                           const int32_t* expert_ends, int E_local, int A,
                                           int M_cap, int H, int I,
                                           const uint8_t* w13_gateup_packed,
                                           const uint8_t* w13_gateup_scale_packed,
                                           float clamp_limit, uint8_t* hq, int32_t* hs,
                                           void* stream) {
  if (I <= 0 || I % 128 != 0) return MOE_ERR_ALIGN;
  float L;
  if (fused_clamp(clamp_limit, L) != MOE_OK) return MOE_ERR_UNSUPPORTED;
  if ((long long)M_cap * I >= (1LL << 31)) return MOE_ERR_SHAPE;
  if (E_local > 0 && M_cap > 0 && (!hq || !hs)) return MOE_ERR_NULL;
  const moe::GemmActOut act{hq, hs, I, L};
  return moe::launch_grouped_gemm(xq, xs, expert_ends, E_local, A, M_cap, H, 2 * I,
                                  w13_gateup_packed, w13_gateup_scale_packed, nullptr, stream,
                                  &act);
}

extern "C" int moe_grouped_gemm1_act_quant_g128(const uint8_t* xq, const int32_t* xs,
                                                const int32_t* expert_ends, int E_local, int A,
                                                int M_cap, int H, int I,
                                                const uint8_t* w13_gateup_packed,
                                                const uint8_t* w13_gateup_scale_packed,
                                                float clamp_limit, uint8_t* hq, int32_t* hs,
                                                void* stream) {
  if (I <= 0 || I % 128 != 0) return MOE_ERR_ALIGN;
  float L;
  if (fused_clamp(clamp_limit, L) != MOE_OK) return MOE_ERR_UNSUPPORTED;
  if ((long long)M_cap * I >= (1LL << 31)) return MOE_ERR_SHAPE;
  if (E_local > 0 && M_cap > 0 && (!hq || !hs)) return MOE_ERR_NULL;
  const moe::GemmActOut act{hq, hs, I, L};
  return moe::launch_grouped_gemm(xq, xs, expert_ends, E_local, A, M_cap, H, 2 * I,
                                  w13_gateup_packed, w13_gateup_scale_packed, nullptr, stream,
                                  &act, true);
}

extern "C" int moe_grouped_gemm1_masked(const uint8_t* xq, const int32_t* xs,
                                        const int32_t* masked_m, int E_local, int m_pad, int H,
                                        int I, const uint8_t* w13_packed,
                                        const uint8_t* w13_scale_packed, uint16_t* gateup,
                                        void* stream) {
  if (I <= 0 || I % 64 != 0) return MOE_ERR_ALIGN;
  int M_cap = 0;
  const int rc = masked_rows(E_local, m_pad, M_cap);
  if (rc != MOE_OK) return rc;
  return moe::launch_grouped_gemm(xq, xs, masked_m, E_local, 1, M_cap, H, 2 * I, w13_packed,
                                  w13_scale_packed, gateup, stream, nullptr, false, m_pad);
}

extern "C" int moe_grouped_gemm2_masked(const uint8_t* hq, const int32_t* hs,
                                        const int32_t* masked_m, int E_local, int m_pad, int I,
                                        int H, const uint8_t* w2_packed,
                                        const uint8_t* w2_scale_packed, uint16_t* down,
                                        void* stream) {
  int M_cap = 0;
  const int rc = masked_rows(E_local, m_pad, M_cap);
  if (rc != MOE_OK) return rc;
  return moe::launch_grouped_gemm(hq, hs, masked_m, E_local, 1, M_cap, I, H, w2_packed,
                                  w2_scale_packed, down, stream, nullptr, false, m_pad);
}

extern "C" int moe_grouped_gemm1_act_quant_masked(const uint8_t* xq, const int32_t* xs,
                                                  const int32_t* masked_m, int E_local, int m_pad,
                                                  int H, int I,
                                                  const uint8_t* w13_gateup_packed,
                                                  const uint8_t* w13_gateup_scale_packed,
                                                  float clamp_limit, uint8_t* hq, int32_t* hs,
                                                  void* stream) {
  if (I <= 0 || I % 128 != 0) return MOE_ERR_ALIGN;
  float L;
  if (fused_clamp(clamp_limit, L) != MOE_OK) return MOE_ERR_UNSUPPORTED;
  int M_cap = 0;
  const int rc = masked_rows(E_local, m_pad, M_cap);
  if (rc != MOE_OK) return rc;
  if ((long long)M_cap * I >= (1LL << 31)) return MOE_ERR_SHAPE;
  if (E_local > 0 && M_cap > 0 && (!hq || !hs)) return MOE_ERR_NULL;
  const moe::GemmActOut act{hq, hs, I, L};
  return moe::launch_grouped_gemm(xq, xs, masked_m, E_local, 1, M_cap, H, 2 * I,
                                  w13_gateup_packed, w13_gateup_scale_packed, nullptr, stream,
                                  &act, false, m_pad);
}

extern "C" int moe_grouped_gemm1_natural(const uint8_t* xq, const int32_t* xs,
                                         const int32_t* expert_ends, int E_local, int A,
                                         int M_cap, int H, int I, const uint8_t* w13,
                                         const uint8_t* w13_scale, uint16_t* gateup,
                                         void* stream) {
  if (I <= 0 || I % 64 != 0) return MOE_ERR_ALIGN;
  return moe::launch_grouped_gemm(xq, xs, expert_ends, E_local, A, M_cap, H, 2 * I, w13,
                                  w13_scale, gateup, stream, nullptr, false, 0, true);
}

extern "C" int moe_grouped_gemm2_natural(const uint8_t* hq, const int32_t* hs,
                                         const int32_t* expert_ends, int E_local, int A,
                                         int M_cap, int I, int H, const uint8_t* w2,
                                         const uint8_t* w2_scale, uint16_t* down, void* stream) {
  return moe::launch_grouped_gemm(hq, hs, expert_ends, E_local, A, M_cap, I, H, w2, w2_scale,
                                  down, stream, nullptr, false, 0, true);
}

extern "C" int moe_grouped_gemm1_act_quant_natural(const uint8_t* xq, const int32_t* xs,
                                                   const int32_t* expert_ends, int E_local, int A,
                                                   int M_cap, int H, int I, const uint8_t* w13,
                                                   const uint8_t* w13_scale, float clamp_limit,
                                                   uint8_t* hq, int32_t* hs, void* stream) {
  if (I <= 0 || I % 128 != 0) return MOE_ERR_ALIGN;
  float L;
  if (fused_clamp(clamp_limit, L) != MOE_OK) return MOE_ERR_UNSUPPORTED;
  if ((long long)M_cap * I >= (1LL << 31)) return MOE_ERR_SHAPE;
  if (E_local > 0 && M_cap > 0 && (!hq || !hs)) return MOE_ERR_NULL;
  const moe::GemmActOut act{hq, hs, I, L};
  return moe::launch_grouped_gemm(xq, xs, expert_ends, E_local, A, M_cap, H, 2 * I, w13,
                                  w13_scale, nullptr, stream, &act, false, 0, true);
}
