// moe_act_quant_liverows: SiLU(gate)*up + FP8/UE8M0 quantisation of the
// live rows of the grouped layout, on gfx950.
//
// "Blackwell FP4 MoE: live-row boundary", sections 1-3: the activation kernel
// receives the same int32 endpoints as the GEMMs, visits only [start, end)
// of each expert and leaves padding unwritten. "Blackwell DeepGEMM FusedMoE
// (sglang)", section 2.4: activation and quantisation are fused so gate/up
// is read once and FP8 + packed scales are written once; SiLU stays fp32.
//
// Work decomposition: the live rows are numbered 0..R-1 in layout order
// (expert by expert, from the endpoints) and split evenly over one block of
// 8 waves per CU, so padding rows are never visited. A block's rows are cut
// into (row, 512-column chunk) items, taken 16 at a time (2 per wave); the
// next batch's loads are issued before the current batch is computed
// (registers double-buffered), so the math of one batch overlaps the loads
// of the next (a block's 48 items at the EP-share shapes are 3 batches per
// wave, where 8-item batches made one batch and no overlap), and the
// sigmoid table's loads go out before any of them. A lane owns 8 consecutive columns of a chunk (16-byte loads
// of gate and up, 8-byte stores of codes), a 32-column group spans 4 lanes
// (amax by two shuffles), a packed scale word spans 16 lanes and is stored
// by its first lane (MN-major).
//
// moe_act_quant_liverows_situ runs the same kernel with the SiTU activation
// of "DeepGEMM FusedMoE on Blackwell (sglang)", section 2.4.1 (situ branch)
// with Kimi-K3's parameters ("Kimi-K3 on SM120 FlashInfer MXFP4"):
//   t = 4 tanh(g/4), v = 25 tanh(u/25), each correctly rounded to fp32 and
//   looked up in LDS by the bf16 pattern (rows of exponents where the value
//   is neither the input itself nor +-b; generated at build time),
//   h = (t * sigma(g)) * v, no clamp.
//
// Arithmetic per element, all IEEE fp32 with no contraction:
//   g = bf16 gate, u = bf16 up; optional clamp g = min(g, L), u = med3(u, -L, L)
//   sig = sigma(g) correctly rounded (looked up in LDS by g's bf16 pattern)
//   h = (g * sig) * u
// and per 32-column group: b = UE8M0 round-up of amax/448, code =
// e4m3_rne(h * 2^(127-b)).
#include <cstring>

#include "common.h"

namespace moe {

// sigma(g) for every bf16 g, generated at build time (gen_sigmoid_table.cpp)
#define MOE_SIGMOID_TABLE_STORAGE __device__ const __attribute__((aligned(16)))
#include "sigmoid_table.inc"
// b*tanh(x/b) for every bf16 x, b = 4 and 25 (gen_situ_table.cpp)
#define MOE_SITU_TABLE_STORAGE __device__ const __attribute__((aligned(16)))
#include "situ_table.inc"
}  // namespace moe
#include "sigmoid_lookup.h"
namespace moe {

// b*tanh(x/b) for a bf16-valued x: x itself below exponent field LO, +-b
// above HI (both checked over every bf16 pattern by the generator), the
// table row in between.
template <int LO, int HI>
__device__ __forceinline__ float scaled_tanh_lookup(const float* tab, float x, float b) {
  const uint32_t bits = __float_as_uint(x) >> 16;   // x is an exact bf16 value
  const int ex = (int)((bits >> 7) & 0xFFu);
  const uint32_t neg = bits >> 15;
  const int idx = (int)neg * ((HI - LO + 1) * 128) + (min(max(ex, LO), HI) - LO) * 128 +
                  (int)(bits & 0x7Fu);
  const float tv = tab[idx];
  return ex < LO ? x : (ex > HI ? (neg ? -b : b) : tv);
}

constexpr int kActThreads = 512;   // 8 waves
constexpr int kActWaves = kActThreads / 64;
constexpr int kActBatch = 2;       // items per wave per batch (double-buffered: small batches
                                   // let one batch's math overlap the next one's loads)
constexpr int kActMaxE = 1024;
constexpr int kActMaxWordsPerRow = 64;  // I <= 8192
// live rows per block (M_cap <= 256 * 12288); the 48 KB this takes also keeps
// the block alone on its CU (over 80 KB of LDS), so that no CU runs two of
// the 256 equal shares
constexpr int kActMaxRowsPerBlock = 12288;
constexpr uint32_t kActOob = 0x80000000u;

__device__ int act_block_scan(int v, int* tmp) {
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

// SITU: the SiTU activation (Kimi-K3's b_s = 4, b_l = 25) instead of SiLU,
// with its two scaled-tanh tables beside the sigmoid table in LDS; no clamp.
// G128: one UE8M0 byte per 128 columns of h instead of per 32, packed four to
// a word over 512 columns ([ceil(I/512)][M_cap] words; bytes of groups past I
// are 0)
// SLAB: the masked slab layout ("DeepGEMM FusedMoE on Blackwell (sglang)",
// section 2.4.2: the varlen act-quant over an (E, m_pad, 2I) slab): expert_ends
// holds masked_m, expert e's live rows are [e slab, e slab + masked_m[e]),
// M_cap = E_local * slab, and the scale words are MN-major per expert
// ([e][word][row - e slab]).
template <bool CLAMP, bool SITU, bool G128, bool SLAB>
__global__ __launch_bounds__(kActThreads, 1) void act_quant_kernel(
    const uint16_t* __restrict__ gateup, const int32_t* __restrict__ expert_ends, int E_local,
    int A, int M_cap, int slab, int I, float L, uint8_t* __restrict__ hq,
    int32_t* __restrict__ hs) {
  __shared__ __attribute__((aligned(16))) float s_tab[MOE_SIGMOID_TABLE_SIZE];
  __shared__ __attribute__((aligned(16))) float s_t4[SITU ? MOE_TANH4_TABLE_SIZE : 4];
  __shared__ __attribute__((aligned(16))) float s_t25[SITU ? MOE_TANH25_TABLE_SIZE : 4];
  __shared__ int s_start[kActMaxE];   // first row of expert e
  __shared__ int s_pref[kActMaxE];    // live rows of the experts before e
  __shared__ int s_tmp[kActWaves];
  __shared__ int s_total;
  __shared__ int s_rows[kActMaxRowsPerBlock];   // row of each of this block's live rows

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  // this thread's two experts' endpoints go out first, then the sigmoid
  // table; loads complete in order, so the scan waits only for the
  // endpoints. Unpredicated (clamped) so that the waits count exactly.
  int endv[2], prevv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = min(2 * tid + j, max(E_local - 1, 0));
    endv[j] = expert_ends[e];
    prevv[j] = expert_ends[max(e - 1, 0)];
  }
  __builtin_amdgcn_sched_barrier(0);     // keep the endpoints ahead of the table
  static_assert(MOE_SIGMOID_TABLE_SIZE % 4 == 0, "table copied as 16-byte vectors");
  constexpr int kVec = MOE_SIGMOID_TABLE_SIZE / 4;
  constexpr int kPer = (kVec + kActThreads - 1) / kActThreads;
  v4i tv[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    // each block starts at its own place in the table, so that the 32 CUs
    // of a cache slice do not all ask for the same lines at once
    int i = tid + j * kActThreads + (int)(blockIdx.x * 97u % (unsigned)kVec);
    i = i >= kVec ? i - kVec : i;
    tv[j] = reinterpret_cast<const v4i*>(g_sigmoid_table)[min(i, kVec - 1)];
  }
  static_assert(MOE_TANH4_TABLE_SIZE % (4 * kActThreads) == 0 &&
                MOE_TANH25_TABLE_SIZE % (4 * kActThreads) == 0, "whole 16-byte vectors per thread");
  constexpr int kPer4 = SITU ? MOE_TANH4_TABLE_SIZE / (4 * kActThreads) : 0;
  constexpr int kPer25 = SITU ? MOE_TANH25_TABLE_SIZE / (4 * kActThreads) : 0;
  v4i t4v[kPer4 > 0 ? kPer4 : 1], t25v[kPer25 > 0 ? kPer25 : 1];
#pragma unroll
  for (int j = 0; j < kPer4; ++j) t4v[j] = reinterpret_cast<const v4i*>(g_tanh4_table)[tid + j * kActThreads];
#pragma unroll
  for (int j = 0; j < kPer25; ++j) t25v[j] = reinterpret_cast<const v4i*>(g_tanh25_table)[tid + j * kActThreads];
  // expert ranges (start_e = align_up(end_{e-1}, A), clamped into [0, M_cap]
  // so that corrupt endpoints cannot leave the buffers) and the exclusive
  // scan of their live-row counts (2 experts per thread)
  int cnt[2], st[2];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = 2 * tid + j;
    if constexpr (SLAB) {
      st[j] = e * slab;
      cnt[j] = e < E_local ? min(max(endv[j], 0), slab) : 0;
    } else {
      const int prev = e == 0 ? 0 : min(max(prevv[j], 0), M_cap);
      const int s0 = min(align_up_dev(prev, A), M_cap);
      const int en = min(max(endv[j], s0), M_cap);
      st[j] = s0;
      cnt[j] = e < E_local ? en - s0 : 0;
    }
    sum += cnt[j];
  }
  int run = act_block_scan(sum, s_tmp);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = 2 * tid + j;
    if (e < E_local) {
      s_start[e] = st[j];
      s_pref[e] = run;
    }
    run += cnt[j];
  }
  if (tid == kActThreads - 1) s_total = run;
  __syncthreads();

  const int R = s_total;
  const int i0 = (int)(((long long)R * blockIdx.x) / gridDim.x);
  const int i1 = (int)(((long long)R * (blockIdx.x + 1)) / gridDim.x);
  const int nrows = min(i1 - i0, kActMaxRowsPerBlock);   // the host guarantees <=
  // row of each of the block's live rows: the expert holding live row i, then its offset
  for (int t = tid; t < nrows; t += kActThreads) {
    const int i = i0 + t;
    int lo = 0, hi = E_local - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= i) lo = mid; else hi = mid - 1;
    }
    s_rows[t] = s_start[lo] + (i - s_pref[lo]);
  }
  __syncthreads();
  const int nchunks = (I + 511) >> 9;
  const float inv_nchunks = 1.0f / (float)nchunks;
  const int items = nrows * nchunks;
  // item -> (local row, chunk) without an integer division (items < 2^24)
  auto split = [&](int it, int& rl, int& ch) {
    int q = (int)((float)it * inv_nchunks);
    int r = it - q * nchunks;
    if (r >= nchunks) { ++q; r -= nchunks; }
    if (r < 0) { --q; r += nchunks; }
    rl = q;
    ch = r;
  };
  const int nbatch = (items + kActWaves * kActBatch - 1) / (kActWaves * kActBatch);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(gateup), (short)0, (int)((uint32_t)M_cap * (uint32_t)(4 * I)), 0x00020000);

  // item it of this block: local live row it / nchunks, chunk it % nchunks.
  // The batch's 8 items are resolved together: lane j < 8 finds item j's
  // row and byte offset (one LDS read for all), then each load takes its
  // offset from that lane.
  auto load_batch = [&](int b, v4i* G, v4i* U) {
    uint32_t my_off = kActOob, my_colb = 0;
    if (lane < kActBatch) {
      const int it = (b * kActBatch + lane) * kActWaves + wid;
      if (it < items) {
        int rl, ch;
        split(it, rl, ch);
        my_colb = (uint32_t)ch * 1024u;                     // chunk start, bytes into the gate half
        my_off = (uint32_t)s_rows[rl] * (uint32_t)(4 * I) + my_colb;
      }
    }
#pragma unroll
    for (int j = 0; j < kActBatch; ++j) {
      const uint32_t base = __builtin_amdgcn_readlane(my_off, j);
      const uint32_t colb = __builtin_amdgcn_readlane(my_colb, j) + (uint32_t)lane * 16u;
      const uint32_t off = (base != kActOob && colb < (uint32_t)I * 2u) ? base + (uint32_t)lane * 16u
                                                                          : kActOob;
      G[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
      U[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off == kActOob ? kActOob : off + (uint32_t)I * 2u, 0, 0);
    }
  };
  auto compute_batch = [&](int b, const v4i* G, const v4i* U) {
#pragma unroll
    for (int j = 0; j < kActBatch; ++j) {
      const int it = (b * kActBatch + j) * kActWaves + wid;
      if (it >= items) break;  // wave-uniform
      int rl, ch;
      split(it, rl, ch);
      const int row = s_rows[rl];
      const int col = ch * 512 + lane * 8;
      const bool act = col < I;
      const uint32_t gw[4] = {(uint32_t)G[j].x, (uint32_t)G[j].y, (uint32_t)G[j].z, (uint32_t)G[j].w};
      const uint32_t uw[4] = {(uint32_t)U[j].x, (uint32_t)U[j].y, (uint32_t)U[j].z, (uint32_t)U[j].w};
      float h[8];
      float amax = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float gv = (q & 1) ? bf16_hi(gw[q >> 1]) : bf16_lo(gw[q >> 1]);
        float uv = (q & 1) ? bf16_hi(uw[q >> 1]) : bf16_lo(uw[q >> 1]);
        if (CLAMP) {
          gv = fminf(gv, L);
          uv = fminf(fmaxf(uv, -L), L);
        }
        const float sig = sigmoid_lookup_table(s_tab, gv);
        if (SITU) {
          // h = fl32(fl32(4 tanh(g/4) * sigma(g)) * 25 tanh(u/25))
          const float t = scaled_tanh_lookup<MOE_TANH4_EXP_LO, MOE_TANH4_EXP_HI>(s_t4, gv, 4.0f);
          const float a = t * sig;
          const float v = scaled_tanh_lookup<MOE_TANH25_EXP_LO, MOE_TANH25_EXP_HI>(s_t25, uv, 25.0f);
          h[q] = a * v;
        } else {
          const float sg = gv * sig;
          h[q] = sg * uv;
        }
        amax = fmaxf(amax, fabsf(h[q]));
      }
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      if constexpr (G128) {               // the 128-column group: 16 lanes
        amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 8, 64));
      }
      const uint32_t bsc = ue8m0_byte_of_amax(amax);
      const float inv = e8m0_reciprocal(bsc);
      uint32_t lo = 0, hi = 0;
      lo = cvt_e4m3x2<false>(h[0] * inv, h[1] * inv, lo);
      lo = cvt_e4m3x2<true>(h[2] * inv, h[3] * inv, lo);
      hi = cvt_e4m3x2<false>(h[4] * inv, h[5] * inv, hi);
      hi = cvt_e4m3x2<true>(h[6] * inv, h[7] * inv, hi);
      uint32_t word;
      if constexpr (G128) {
        // byte q of the chunk's word: the group of lanes 16q .. 16q + 15
        const bool in = ch * 512 + 128 * (lane >> 4) < I;
        word = (in ? bsc : 0u) << (8 * (lane >> 4));
        word |= __shfl_xor(word, 16, 64);
        word |= __shfl_xor(word, 32, 64);
      } else {
        word = bsc << (8 * ((lane >> 2) & 3));
        word |= __shfl_xor(word, 4, 64);
        word |= __shfl_xor(word, 8, 64);
      }
      if (act) {
        *reinterpret_cast<uint2*>(hq + (size_t)row * I + col) = make_uint2(lo, hi);
        // scale word w of the row: [w][row] over the whole buffer, or
        // [e][w][row - e slab] inside expert e's slab
        size_t hs0 = row;
        int hss = M_cap;
        if constexpr (SLAB) {
          const int WN = G128 ? (I + 511) >> 9 : I >> 7;
          hs0 = (size_t)(row / slab) * (size_t)(WN - 1) * (size_t)slab + row;
          hss = slab;
        }
        if constexpr (G128) {
          if (lane == 0) hs[hs0 + (size_t)ch * hss] = (int32_t)word;
        } else {
          if ((lane & 15) == 0) hs[hs0 + (size_t)(col >> 7) * hss] = (int32_t)word;
        }
      }
    }
  };

  // batch loads are unconditional (items past the end read out of range,
  // which returns zeros and touches no memory), so every wait counts loads
  // exactly: the table's stores below wait only for the table
  v4i GA[kActBatch], UA[kActBatch], GB[kActBatch], UB[kActBatch];
  load_batch(0, GA, UA);
  // the table goes to LDS while the first batch is in flight (it waits only
  // for the table's own loads, which were issued first)
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    int i = tid + j * kActThreads + (int)(blockIdx.x * 97u % (unsigned)kVec);
    i = i >= kVec ? i - kVec : i;
    if (tid + j * kActThreads < kVec) reinterpret_cast<v4i*>(s_tab)[i] = tv[j];
  }
#pragma unroll
  for (int j = 0; j < kPer4; ++j) reinterpret_cast<v4i*>(s_t4)[tid + j * kActThreads] = t4v[j];
#pragma unroll
  for (int j = 0; j < kPer25; ++j) reinterpret_cast<v4i*>(s_t25)[tid + j * kActThreads] = t25v[j];
  __syncthreads();
  for (int b = 0; b < nbatch; b += 2) {
    load_batch(b + 1, GB, UB);
    compute_batch(b, GA, UA);
    if (b + 1 >= nbatch) break;
    load_batch(b + 2, GA, UA);
    compute_batch(b + 1, GB, UB);
  }
}

}  // namespace moe

namespace {

// shapes and limits shared by the SiLU and SiTU entry points
int act_quant_check(const uint16_t* gateup, const int32_t* expert_ends, int E_local, int A,
                    int M_cap, int I, uint8_t* hq, int32_t* hs) {
  using namespace moe;
  if (E_local < 0 || E_local > kActMaxE || A < 1 || M_cap < 0 || I <= 0) return MOE_ERR_SHAPE;
  if (I % 128 != 0 || M_cap % 4 != 0) return MOE_ERR_ALIGN;
  if (I / 128 > kActMaxWordsPerRow) return MOE_ERR_SHAPE;
  // one buffer range covers gate/up: M_cap rows of 4*I bytes below 2 GiB;
  // at most kActMaxRowsPerBlock live rows per block
  if ((long long)M_cap * I * 4 >= (1LL << 31)) return MOE_ERR_SHAPE;
  if (M_cap > 256 * kActMaxRowsPerBlock) return MOE_ERR_SHAPE;
  if (E_local == 0 || M_cap == 0) return MOE_OK;
  if (!gateup || !expert_ends || !hq || !hs) return MOE_ERR_NULL;
  return 1;   // launch
}

}  // namespace

namespace moe {
// slab > 0: the masked slab layout (expert_ends = masked_m, M_cap = E_local
// * slab; group 32 only)
static int act_quant_silu(const uint16_t* gateup, const int32_t* expert_ends, int E_local, int A,
                          int M_cap, int I, float clamp_limit, uint8_t* hq, int32_t* hs,
                          void* stream, bool g128, int slab = 0) {
  bool clamp = false;
  if (clamp_limit > 0.f && clamp_limit < __builtin_inff()) {
    uint32_t bits;
    std::memcpy(&bits, &clamp_limit, 4);
    if (bits & 0xFFFFu) return MOE_ERR_UNSUPPORTED;  // the limit must be an exact bf16 value
    clamp = true;
  } else if (!(clamp_limit <= 0.f) && !(clamp_limit == __builtin_inff())) {
    return MOE_ERR_UNSUPPORTED;  // NaN
  }
  const int rc = act_quant_check(gateup, expert_ends, E_local, A, M_cap, I, hq, hs);
  if (rc <= 0) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int grid = 256;         // one block per CU; each takes 1/256 of the live rows
  auto kernel = clamp ? (g128 ? act_quant_kernel<true, false, true, false>
                             : act_quant_kernel<true, false, false, false>)
                     : (g128 ? act_quant_kernel<false, false, true, false>
                             : act_quant_kernel<false, false, false, false>);
  if (slab > 0)
    kernel = clamp ? act_quant_kernel<true, false, false, true> : act_quant_kernel<false, false, false, true>;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kActThreads), 0, st, gateup, expert_ends, E_local, A,
                     M_cap, slab, I, clamp ? clamp_limit : 0.f, hq, hs);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
}  // namespace moe

extern "C" int moe_act_quant_liverows(const uint16_t* gateup, const int32_t* expert_ends,
                                      int E_local, int A, int M_cap, int I, float clamp_limit,
                                      uint8_t* hq, int32_t* hs, void* stream) {
  return moe::act_quant_silu(gateup, expert_ends, E_local, A, M_cap, I, clamp_limit, hq, hs,
                             stream, false);
}

extern "C" int moe_act_quant_liverows_g128(const uint16_t* gateup, const int32_t* expert_ends,
                                           int E_local, int A, int M_cap, int I,
                                           float clamp_limit, uint8_t* hq, int32_t* hs,
                                           void* stream) {
  return moe::act_quant_silu(gateup, expert_ends, E_local, A, M_cap, I, clamp_limit, hq, hs,
                             stream, true);
}

extern "C" int moe_act_quant_liverows_situ(const uint16_t* gateup, const int32_t* expert_ends,
                                           int E_local, int A, int M_cap, int I, float situ_beta,
                                           float situ_linear_beta, uint8_t* hq, int32_t* hs,
                                           void* stream) {
  using namespace moe;
  // the scaled-tanh tables are built for Kimi-K3's parameters only
  if (situ_beta != 4.0f || situ_linear_beta != 25.0f) return MOE_ERR_UNSUPPORTED;
  const int rc = act_quant_check(gateup, expert_ends, E_local, A, M_cap, I, hq, hs);
  if (rc <= 0) return rc;
  hipLaunchKernelGGL((act_quant_kernel<false, true, false, false>), dim3(256), dim3(kActThreads), 0,
                     (hipStream_t)stream, gateup, expert_ends, E_local, A, M_cap, 0, I, 0.f, hq, hs);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_act_quant_masked(const uint16_t* gateup, const int32_t* masked_m, int E_local,
                                    int m_pad, int I, float clamp_limit, uint8_t* hq, int32_t* hs,
                                    void* stream) {
  if (E_local < 0 || m_pad < 0) return MOE_ERR_SHAPE;
  if (m_pad % 4 != 0) return MOE_ERR_ALIGN;
  if ((long long)E_local * m_pad >= (1LL << 31)) return MOE_ERR_SHAPE;
  return moe::act_quant_silu(gateup, masked_m, E_local, 1, E_local * m_pad, I, clamp_limit, hq, hs,
                             stream, false, m_pad);
}
