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
// and it computes every slot routed to that expert, so each selected
// expert's weights are read once per call instead of once per slot. The
// slot ids are copied to LDS in one parallel load and the duplicate test
// runs there. A wave owns 8 weight rows (4 output columns: 4 gate + 4 up
// rows when the GLU is fused; else 8 output columns) and issues all their
// 16-byte chunks (strided by the wave over K) before the activations of the
// expert's slots are staged in LDS as bf16, so the two loads overlap; each
// chunk is converted to exact bf16 pairs and accumulated with bf16 dot
// products in fp32 against the LDS activations, and the 64 partial sums of
// a row are folded by shuffles. With the GLU fused, the GLU is applied to
// the bf16-rounded gate and up results before the single bf16 store.
#include <cmath>

#include "common.h"

namespace moe {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / 64;
constexpr int kGemvRows = 8;          // weight rows per wave (GLU: 4 gate + 4 up)
constexpr int kGemvMaxSlots = 64;     // T*k
constexpr int kGemvSlotBatch = 8;     // slots whose activations are staged in LDS at once
constexpr int kGemvMaxChunks = 4;     // 16-byte weight chunks per lane and row (K <= 4096 FP8)

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float glu_apply(float g, float u, float alpha, float beta, float limit) {
  if (limit > 0.f) {
    g = fminf(g, limit);
    u = fminf(fmaxf(u, -limit), limit);
  }
  const float sig = 1.0f / (1.0f + expf(-alpha * g));
  return g * sig * (u + beta);
}

// 16 weight bytes -> bf16 pairs (exact: E4M3 and E2M1 values fit bf16).
// FP8: 16 weights -> 8 pairs; MXFP4: 32 weights -> 16 pairs (low nibble first).
template <bool MXFP4>
__device__ __forceinline__ void weights_to_bf16(const v4i raw, v2bf* wp) {
  const uint32_t d[4] = {(uint32_t)raw.x, (uint32_t)raw.y, (uint32_t)raw.z, (uint32_t)raw.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (MXFP4) {
      wp[4 * q + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[q], 1.0f, 0);
      wp[4 * q + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[q], 1.0f, 1);
      wp[4 * q + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[q], 1.0f, 2);
      wp[4 * q + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[q], 1.0f, 3);
    } else {
      wp[2 * q + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[q], 1.0f, false);
      wp[2 * q + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[q], 1.0f, true);
    }
  }
}

template <bool MXFP4, bool GLU, int CH>
__global__ __launch_bounds__(kGemvThreads) void sparse_gemv_kernel(
    const uint16_t* __restrict__ act, int act_per_slot, const int32_t* __restrict__ ids, int T,
    int k, int expert_start, int E_local, int N, int K, const uint8_t* __restrict__ W,
    const void* __restrict__ w_scale, const uint16_t* __restrict__ bias, float alpha,
    float beta, float limit, uint16_t* __restrict__ out, int32_t* __restrict__ slot_row) {
  extern __shared__ __attribute__((aligned(16))) uint16_t s_act[];  // [kGemvSlotBatch][K] bf16

  const int q = blockIdx.y;  // flattened slot t*k+s
  const int tid = threadIdx.x;
  const int lane = tid & 63;
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
  uint64_t slot_mask = same;                  // slots p >= q routed to this expert

  const int wid = tid >> 6;
  const int n_out = GLU ? N / 2 : N;
  constexpr int kOuts = GLU ? kGemvRows / 2 : kGemvRows;    // output columns per wave
  const int col0 = (blockIdx.x * kGemvWaves + wid) * kOuts;
  const size_t row_bytes = MXFP4 ? (size_t)K / 2 : (size_t)K;
  const int kchunk = MXFP4 ? 32 : 16;  // weights per 16-byte chunk
  const int nchunks = K / kchunk;
  const uint8_t* We = W + (size_t)e * N * row_bytes;
  const float fp8_scale = MXFP4 ? 1.f : reinterpret_cast<const float*>(w_scale)[e];
  const uint8_t* Ws = MXFP4 ? reinterpret_cast<const uint8_t*>(w_scale) + (size_t)e * N * (K / 32)
                            : nullptr;
  // weight row of register row r (clamped into range; columns past n_out
  // are computed and never stored)
  auto row_of = [&](int r) {
    if (GLU) return min(col0 + (r % kOuts), n_out - 1) + (r < kOuts ? 0 : N / 2);
    return min(col0 + r, N - 1);
  };

  // every weight chunk of this wave's rows goes out first
  v4i raw[kGemvRows][CH];
  float gsc[kGemvRows][CH];
#pragma unroll
  for (int r = 0; r < kGemvRows; ++r) {
    const uint8_t* wr = We + (size_t)row_of(r) * row_bytes;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = lane + 64 * c;
      raw[r][c] = v4i{0, 0, 0, 0};
      gsc[r][c] = 0.f;
      if (ch < nchunks) {
        raw[r][c] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wr + (size_t)ch * 16));
        if (MXFP4) gsc[r][c] = e8m0_value(Ws[(size_t)row_of(r) * (K / 32) + ch]);
      }
    }
  }
  const int nslots = __popcll(slot_mask);
  // slot number of the i-th set bit of slot_mask (i < nslots)
  auto nth_slot = [&](int i) {
    uint64_t m = slot_mask;
    for (int j = 0; j < i; ++j) m &= m - 1ull;
    return __ffsll((unsigned long long)m) - 1;
  };

  for (int sb = 0; sb < nslots; sb += kGemvSlotBatch) {
    const int S = min(kGemvSlotBatch, nslots - sb);
    if (sb > 0) __syncthreads();   // the previous batch is done with s_act
    for (int i = tid; i < S * (K / 8); i += kGemvThreads) {
      const int s = i / (K / 8), c8 = i - s * (K / 8);
      const int p = nth_slot(sb + s);
      const int arow = act_per_slot ? p : p / k;
      reinterpret_cast<v4i*>(s_act + (size_t)s * K)[c8] =
          reinterpret_cast<const v4i*>(act + (size_t)arow * K)[c8];
    }
    __syncthreads();

    // one slot at a time: 8 row accumulators live, the weights stay in
    // registers and are converted again for every slot
    for (int s = 0; s < S; ++s) {
      float acc[kGemvRows];
#pragma unroll
      for (int r = 0; r < kGemvRows; ++r) acc[r] = 0.f;
      const uint16_t* as = s_act + (size_t)s * K;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int ch = lane + 64 * c;
        if (ch >= nchunks) break;
        const v2bf* ap = reinterpret_cast<const v2bf*>(as + ch * kchunk);
        v2bf av[MXFP4 ? 16 : 8];
#pragma unroll
        for (int i = 0; i < (MXFP4 ? 16 : 8); ++i) av[i] = ap[i];
#pragma unroll
        for (int r = 0; r < kGemvRows; ++r) {
          v2bf wp[16];
          weights_to_bf16<MXFP4>(raw[r][c], wp);
          float part = 0.f;
#pragma unroll
          for (int i = 0; i < (MXFP4 ? 16 : 8); ++i)
            part = __builtin_amdgcn_fdot2_f32_bf16(wp[i], av[i], part, false);
          acc[r] = MXFP4 ? fmaf(part, gsc[r][c], acc[r]) : acc[r] + part;
        }
      }
      // fold, epilogue (scale, bias, bf16), GLU, store
      const int p = nth_slot(sb + s);
#pragma unroll
      for (int r = 0; r < kOuts; ++r) {
        const int j = col0 + r;
        float y[2];
#pragma unroll
        for (int hf = 0; hf < (GLU ? 2 : 1); ++hf) {
          const int rr = r + hf * kOuts;
          const int n = row_of(rr);
          const float bv = bias ? bf16_to_f32(bias[(size_t)e * N + n]) : 0.f;
          const float tot = wave_sum_f32(acc[rr]);
          const float yv = MXFP4 ? __fadd_rn(tot, bv) : __fadd_rn(__fmul_rn(tot, fp8_scale), bv);
          y[hf] = bf16_to_f32((uint16_t)f32_to_bf16_bits(yv));
        }
        if (lane == 0 && j < n_out) {
          const float v = GLU ? glu_apply(y[0], y[1], alpha, beta, limit) : y[0];
          out[(size_t)p * n_out + j] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
    }
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
  if (K % (wfmt == MOE_W_MXFP4_G32 ? 32 : 16) != 0) return MOE_ERR_ALIGN;
  if (K % 8 != 0) return MOE_ERR_ALIGN;
  if (glu && N % 2 != 0) return MOE_ERR_ALIGN;
  if (act_per_slot != 0 && act_per_slot != 1) return MOE_ERR_UNSUPPORTED;
  const size_t lds = (size_t)kGemvSlotBatch * K * sizeof(uint16_t);
  const int kchunk = wfmt == MOE_W_MXFP4_G32 ? 32 : 16;
  const int chunks_per_lane = (K / kchunk + 63) / 64;
  if (chunks_per_lane > kGemvMaxChunks) return MOE_ERR_SHAPE;  // K <= 4096 (FP8) / 8192 (MXFP4)
  if (lds > 64 * 1024) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!act || !topk_ids || !w || !w_scale || !out) return MOE_ERR_NULL;
  const int n_out = glu ? N / 2 : N;
  const int outs_per_block = kGemvWaves * (glu ? kGemvRows / 2 : kGemvRows);
  dim3 grid((n_out + outs_per_block - 1) / outs_per_block, T * k);
  hipStream_t st = (hipStream_t)stream;
#define MOE_GEMV_LAUNCH(MX, G, CHN)                                                             \
  hipLaunchKernelGGL((sparse_gemv_kernel<MX, G, CHN>), grid, dim3(kGemvThreads), lds, st, act,  \
                     act_per_slot, topk_ids, T, k, expert_start, E_local, N, K, w, w_scale, bias, \
                     glu_alpha, glu_beta, glu_limit, out, slot_row)
#define MOE_GEMV_CH(MX, G)                       \
  switch (chunks_per_lane) {                     \
    case 1: MOE_GEMV_LAUNCH(MX, G, 1); break;    \
    case 2: MOE_GEMV_LAUNCH(MX, G, 2); break;    \
    case 3: MOE_GEMV_LAUNCH(MX, G, 3); break;    \
    default: MOE_GEMV_LAUNCH(MX, G, 4); break;   \
  }
  const bool mx = wfmt == MOE_W_MXFP4_G32;
  if (mx && glu) MOE_GEMV_CH(true, true)
  else if (mx) MOE_GEMV_CH(true, false)
  else if (glu) MOE_GEMV_CH(false, true)
  else MOE_GEMV_CH(false, false)
#undef MOE_GEMV_CH
#undef MOE_GEMV_LAUNCH
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
