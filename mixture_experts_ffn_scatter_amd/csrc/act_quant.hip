// moe_act_quant_liverows: SiLU(gate)*up + FP8/UE8M0 quantisation of the
// live rows of the grouped layout, on gfx950.
//
// "Blackwell FP4 MoE: live-row boundary", sections 1-3: the activation kernel
// receives the same int32 endpoints as the GEMMs, visits only [start, end)
// of each expert and leaves padding unwritten. "Blackwell DeepGEMM FusedMoE
// (sglang)", section 2.4: activation and quantisation are fused so gate/up
// is read once and FP8 + packed scales are written once; SiLU stays fp32.
//
// Work decomposition: one persistent block of 8 waves per CU walks units of
// [0, end of the last expert). A unit is up to 32 (row, 512-column chunk)
// items (rows per unit = 32 / chunks per row, at most 16); a row is
// processed only if it lies inside some [start_e, end_e). A lane owns 8
// consecutive columns of a chunk (16-byte loads of gate and up, 8-byte
// stores of codes), a 32-column group spans 4 lanes (amax by two shuffles),
// a packed scale word spans 16 lanes. The unit's scale words are staged in
// LDS and stored MN-major as one contiguous run per scale row. The next
// unit's loads are issued before the current unit is computed (registers
// double-buffered); loads go through a buffer resource that ends at the
// unit's last row, and items that are dead or past the row read nothing, so
// every wave issues the same load stream and padding is never read.
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

constexpr int kActThreads = 512;   // 8 waves
constexpr int kActWaves = kActThreads / 64;
constexpr int kActItems = 32;      // (row, 512-column chunk) items per unit
constexpr int kActBatch = kActItems / kActWaves;
constexpr int kActMaxRows = 16;
constexpr int kActMaxE = 1024;
constexpr int kActMaxWordsPerRow = 64;  // I <= 8192
constexpr uint32_t kActOob = 0x80000000u;

__device__ __forceinline__ float sigmoid_lookup(const float* tab, float g) {
  const uint32_t bits = __float_as_uint(g) >> 16;  // g is an exact bf16 value
  uint32_t a = bits & 0x7FFFu;
  a = min(max(a, (uint32_t)(MOE_SIGMOID_EXP_LO << 7)), (uint32_t)((MOE_SIGMOID_EXP_HI << 7) | 127));
  const uint32_t idx = a - (MOE_SIGMOID_EXP_LO << 7) +
                       ((bits >> 15) ? (uint32_t)((MOE_SIGMOID_EXP_HI - MOE_SIGMOID_EXP_LO + 1) * 128) : 0u);
  return tab[idx];
}

// largest e with start_e <= r (starts are non-decreasing; an expert sharing
// its start with a later one is empty)
__device__ __forceinline__ int expert_of_row(const int* s_start, int E, int r) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_start[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <bool CLAMP>
__global__ __launch_bounds__(kActThreads, 1) void act_quant_kernel(
    const uint16_t* __restrict__ gateup, const int32_t* __restrict__ expert_ends, int E_local,
    int A, int M_cap, int I, float L, uint8_t* __restrict__ hq, int32_t* __restrict__ hs) {
  __shared__ __attribute__((aligned(16))) float s_tab[MOE_SIGMOID_TABLE_SIZE];
  __shared__ int s_start[kActMaxE];
  __shared__ int s_end[kActMaxE];
  __shared__ uint32_t s_words[2][kActMaxWordsPerRow * kActMaxRows];
  __shared__ int s_live[2][kActMaxRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  // the sigmoid table's loads go out first (loads complete in order)
  static_assert(MOE_SIGMOID_TABLE_SIZE % 4 == 0, "table copied as 16-byte vectors");
  constexpr int kVec = MOE_SIGMOID_TABLE_SIZE / 4;
  constexpr int kPer = (kVec + kActThreads - 1) / kActThreads;
  v4i tv[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = tid + j * kActThreads;
    tv[j] = i < kVec ? reinterpret_cast<const v4i*>(g_sigmoid_table)[i] : v4i{0, 0, 0, 0};
  }
  for (int e = tid; e < E_local; e += kActThreads) {
    int s, en;
    expert_range(expert_ends, e, A, M_cap, s, en);
    s_start[e] = s;
    s_end[e] = en;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = tid + j * kActThreads;
    if (i < kVec) reinterpret_cast<v4i*>(s_tab)[i] = tv[j];
  }
  __syncthreads();
  // ends are monotone in a valid layout; the running max keeps the walk
  // bounded by the farthest end even for inconsistent metadata
  int last = 0;
  for (int e = 0; e < E_local; ++e) last = max(last, s_end[e]);
  const int words = I >> 7;
  const int nchunks = (I + 511) >> 9;
  const int R = min(kActMaxRows, max(1, kActItems / nchunks));   // rows per unit
  const int items = R * nchunks;
  const int n_units = (last + R - 1) / R;

  auto live_of = [&](int unit, int buf) {
    if (tid < R) {
      const int r = unit * R + tid;
      bool live = false;
      if (r < last) {
        const int e = expert_of_row(s_start, E_local, r);
        live = r >= s_start[e] && r < s_end[e];
      }
      s_live[buf][tid] = live ? 1 : 0;
    }
  };
  // gate/up of this wave's items of a unit; dead items read nothing
  auto load_unit = [&](int unit, int buf, v4i* G, v4i* U) {
    const int r0 = unit * R;
    const int nrows = min(R, last - r0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(gateup + (size_t)r0 * (2 * I)), (short)0,
        (int)((uint32_t)max(nrows, 0) * (uint32_t)(4 * I)), 0x00020000);
#pragma unroll
    for (int b = 0; b < kActBatch; ++b) {
      const int it = wid + b * kActWaves;
      const int rl = it / nchunks;
      const int col = (it - rl * nchunks) * 512 + lane * 8;
      const bool ok = it < items && col < I && s_live[buf][rl < R ? rl : 0];
      const uint32_t off = (uint32_t)rl * (uint32_t)(4 * I) + (uint32_t)col * 2u;
      G[b] = __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? off : kActOob, 0, 0);
      U[b] = __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? off + (uint32_t)I * 2u : kActOob, 0, 0);
    }
  };
  auto compute_unit = [&](int unit, int buf, const v4i* G, const v4i* U) {
    const int r0 = unit * R;
#pragma unroll
    for (int b = 0; b < kActBatch; ++b) {
      const int it = wid + b * kActWaves;
      if (it >= items) break;  // wave-uniform
      const int rl = it / nchunks;
      if (!s_live[buf][rl]) continue;  // wave-uniform
      const int col = (it - rl * nchunks) * 512 + lane * 8;
      const bool act = col < I;
      const uint32_t gw[4] = {(uint32_t)G[b].x, (uint32_t)G[b].y, (uint32_t)G[b].z, (uint32_t)G[b].w};
      const uint32_t uw[4] = {(uint32_t)U[b].x, (uint32_t)U[b].y, (uint32_t)U[b].z, (uint32_t)U[b].w};
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
        const float sig = sigmoid_lookup(s_tab, gv);
        const float sg = gv * sig;
        h[q] = sg * uv;
        amax = fmaxf(amax, fabsf(h[q]));
      }
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      const uint32_t bsc = ue8m0_ceil_byte(amax / 448.0f);
      const float inv = e8m0_reciprocal(bsc);
      uint32_t lo = 0, hi = 0;
      lo = cvt_e4m3x2<false>(h[0] * inv, h[1] * inv, lo);
      lo = cvt_e4m3x2<true>(h[2] * inv, h[3] * inv, lo);
      hi = cvt_e4m3x2<false>(h[4] * inv, h[5] * inv, hi);
      hi = cvt_e4m3x2<true>(h[6] * inv, h[7] * inv, hi);
      uint32_t word = bsc << (8 * ((lane >> 2) & 3));
      word |= __shfl_xor(word, 4, 64);
      word |= __shfl_xor(word, 8, 64);
      if (act) {
        *reinterpret_cast<uint2*>(hq + (size_t)(r0 + rl) * I + col) = make_uint2(lo, hi);
        if ((lane & 15) == 0) s_words[buf][(col >> 7) * kActMaxRows + rl] = word;
      }
    }
  };
  auto store_words = [&](int unit, int buf) {
    const int r0 = unit * R;
    for (int i = tid; i < words * R; i += kActThreads) {
      const int c = i / R;
      const int rl = i - c * R;
      if (s_live[buf][rl]) hs[(size_t)c * M_cap + r0 + rl] = (int32_t)s_words[buf][c * kActMaxRows + rl];
    }
  };
  // one unit: prefetch the next one, compute this one, store its words
  auto step = [&](int unit, int buf, const v4i* Gc, const v4i* Uc, v4i* Gn, v4i* Un) {
    const int un = unit + gridDim.x;
    __syncthreads();   // the previous unit's word stores are done with the other buffer
    if (un < n_units) live_of(un, buf ^ 1);
    __syncthreads();
    if (un < n_units) load_unit(un, buf ^ 1, Gn, Un);
    compute_unit(unit, buf, Gc, Uc);
    __syncthreads();
    store_words(unit, buf);
    return un;
  };

  v4i GA[kActBatch], UA[kActBatch], GB[kActBatch], UB[kActBatch];
  int unit = blockIdx.x;
  if (unit < n_units) live_of(unit, 0);
  __syncthreads();
  if (unit < n_units) load_unit(unit, 0, GA, UA);
  while (unit < n_units) {
    unit = step(unit, 0, GA, UA, GB, UB);
    if (unit >= n_units) break;
    unit = step(unit, 1, GB, UB, GA, UA);
  }
}

}  // namespace moe

extern "C" int moe_act_quant_liverows(const uint16_t* gateup, const int32_t* expert_ends,
                                      int E_local, int A, int M_cap, int I, float clamp_limit,
                                      uint8_t* hq, int32_t* hs, void* stream) {
  using namespace moe;
  if (E_local < 0 || E_local > kActMaxE || A < 1 || M_cap < 0 || I <= 0) return MOE_ERR_SHAPE;
  if (I % 128 != 0 || M_cap % 4 != 0) return MOE_ERR_ALIGN;
  if (I / 128 > kActMaxWordsPerRow) return MOE_ERR_SHAPE;
  bool clamp = false;
  if (clamp_limit > 0.f && clamp_limit < __builtin_inff()) {
    uint32_t bits;
    std::memcpy(&bits, &clamp_limit, 4);
    if (bits & 0xFFFFu) return MOE_ERR_UNSUPPORTED;  // the limit must be an exact bf16 value
    clamp = true;
  } else if (!(clamp_limit <= 0.f) && !(clamp_limit == __builtin_inff())) {
    return MOE_ERR_UNSUPPORTED;  // NaN
  }
  if (E_local == 0 || M_cap == 0) return MOE_OK;
  if (!gateup || !expert_ends || !hq || !hs) return MOE_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  // one persistent block per CU (the sigmoid table takes 33 KB of LDS per
  // block, loaded once and reused for every unit the block walks)
  const int max_units = M_cap;   // at least one row per unit
  const int grid = max_units < 256 ? max_units : 256;
  if (clamp)
    hipLaunchKernelGGL(act_quant_kernel<true>, dim3(grid), dim3(kActThreads), 0, st, gateup,
                       expert_ends, E_local, A, M_cap, I, clamp_limit, hq, hs);
  else
    hipLaunchKernelGGL(act_quant_kernel<false>, dim3(grid), dim3(kActThreads), 0, st, gateup,
                       expert_ends, E_local, A, M_cap, I, 0.f, hq, hs);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
