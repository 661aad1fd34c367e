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
// activations of those slots are staged in LDS as fp32. A wave computes
// 8 output columns (or 8 gate/up row pairs when the GLU is fused); a lane
// covers 16-byte weight chunks strided by the wave, and the 64 partial sums
// of a column are folded by shuffles. With the GLU fused, gate row j and up
// row j + N/2 are computed by the same wave and the GLU is applied to their
// bf16-rounded results before the single bf16 store.
#include <cmath>

#include "common.h"

namespace moe {

constexpr int kGemvThreads = 256;
constexpr int kGemvColsPerWave = 8;
constexpr int kGemvColsPerBlock = kGemvColsPerWave * (kGemvThreads / 64);
constexpr int kGemvMaxSlots = 64;  // T*k
constexpr int kGemvSlotBatch = 4;  // slots staged in LDS at once

__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  // sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const uint32_t mag = e == 0u ? (m ? 0x3F000000u : 0u) : (((e + 126u) << 23) | (m << 22));
  return __uint_as_float(mag | ((c & 8u) << 28));
}

__device__ __forceinline__ float glu_apply(float g, float u, float alpha, float beta, float limit) {
  if (limit > 0.f) {
    g = fminf(g, limit);
    u = fminf(fmaxf(u, -limit), limit);
  }
  const float sig = 1.0f / (1.0f + expf(-alpha * g));
  return g * sig * (u + beta);
}

template <bool MXFP4, bool GLU>
__global__ __launch_bounds__(kGemvThreads) void sparse_gemv_kernel(
    const uint16_t* __restrict__ act, int act_per_slot, const int32_t* __restrict__ ids, int T,
    int k, int expert_start, int E_local, int N, int K, const uint8_t* __restrict__ W,
    const void* __restrict__ w_scale, const uint16_t* __restrict__ bias, float alpha,
    float beta, float limit, uint16_t* __restrict__ out, int32_t* __restrict__ slot_row) {
  extern __shared__ float s_act[];  // [kGemvSlotBatch][K]
  __shared__ int s_slots[kGemvMaxSlots];
  __shared__ int s_nslots;

  const int q = blockIdx.y;  // flattened slot t*k+s
  const int tid = threadIdx.x;
  const int nq = T * k;
  const int id = ids[q];
  const int e = id - expert_start;
  const bool local = e >= 0 && e < E_local;
  if (blockIdx.x == 0 && tid == 0 && slot_row) slot_row[q] = local ? q : -1;
  if (!local) return;  // block-uniform
  // the first slot of each distinct local expert does the work
  for (int p = 0; p < q; ++p)
    if (ids[p] == id) return;  // block-uniform (same loop in every thread)
  if (tid == 0) {
    int n = 0;
    for (int p = q; p < nq; ++p)
      if (ids[p] == id) s_slots[n++] = p;
    s_nslots = n;
  }
  __syncthreads();
  const int nslots = s_nslots;

  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int n_out = GLU ? N / 2 : N;
  const int col0 = blockIdx.x * kGemvColsPerBlock + wid * kGemvColsPerWave;
  const size_t row_bytes = MXFP4 ? (size_t)K / 2 : (size_t)K;
  const uint8_t* We = W + (size_t)e * N * row_bytes;
  const float fp8_scale = MXFP4 ? 1.f : reinterpret_cast<const float*>(w_scale)[e];
  const uint8_t* Ws = MXFP4 ? reinterpret_cast<const uint8_t*>(w_scale) + (size_t)e * N * (K / 32)
                            : nullptr;
  constexpr int rows_per_col = GLU ? 2 : 1;
  const int kchunk = MXFP4 ? 32 : 16;  // weights per 16-byte chunk
  const int nchunks = K / kchunk;

  for (int sb = 0; sb < nslots; sb += kGemvSlotBatch) {
    const int S = min(kGemvSlotBatch, nslots - sb);
    __syncthreads();
    for (int i = tid; i < S * K; i += kGemvThreads) {
      const int s = i / K, kk = i - s * K;
      const int p = s_slots[sb + s];
      const int arow = act_per_slot ? p : p / k;
      s_act[i] = bf16_to_f32(act[(size_t)arow * K + kk]);
    }
    __syncthreads();

    for (int c = 0; c < kGemvColsPerWave; ++c) {
      const int j = col0 + c;
      if (j >= n_out) break;  // wave-uniform
      float y[2][kGemvSlotBatch];
#pragma unroll
      for (int r = 0; r < rows_per_col; ++r) {
        const int n = j + r * (N / 2);
        const uint8_t* wr = We + (size_t)n * row_bytes;
        float accs[kGemvSlotBatch];
#pragma unroll
        for (int s = 0; s < kGemvSlotBatch; ++s) accs[s] = 0.f;
        for (int ch = lane; ch < nchunks; ch += 64) {
          const uint4 raw = *reinterpret_cast<const uint4*>(wr + (size_t)ch * 16);
          const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
          float wf[32];
          if (MXFP4) {
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
              for (int nb = 0; nb < 8; ++nb) wf[d * 8 + nb] = e2m1_to_f32((wv[d] >> (4 * nb)) & 0xFu);
          } else {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const v2f p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[d], false);
              const v2f p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)wv[d], true);
              wf[d * 4 + 0] = p0.x;
              wf[d * 4 + 1] = p0.y;
              wf[d * 4 + 2] = p1.x;
              wf[d * 4 + 3] = p1.y;
            }
          }
          const int kb = ch * kchunk;
          const float gscale = MXFP4 ? e8m0_value(Ws[(size_t)n * (K / 32) + ch]) : 1.f;
#pragma unroll
          for (int s = 0; s < kGemvSlotBatch; ++s) {
            if (s < S) {
              const float* a = s_act + s * K + kb;
              float part = 0.f;
#pragma unroll
              for (int i = 0; i < (MXFP4 ? 32 : 16); ++i) part = fmaf(wf[i], a[i], part);
              accs[s] = fmaf(part, gscale, accs[s]);
            }
          }
        }
#pragma unroll
        for (int s = 0; s < kGemvSlotBatch; ++s) {
          if (s < S) {
            const float tot = wave_sum_f32(accs[s]);
            const float bv = bias ? bf16_to_f32(bias[(size_t)e * N + n]) : 0.f;
            const float yv = MXFP4 ? __fadd_rn(tot, bv) : __fadd_rn(__fmul_rn(tot, fp8_scale), bv);
            y[r][s] = bf16_to_f32((uint16_t)f32_to_bf16_bits(yv));
          }
        }
      }
      if (lane == 0) {
#pragma unroll
        for (int s = 0; s < kGemvSlotBatch; ++s) {
          if (s >= S) break;
          const int p = s_slots[sb + s];
          float v = y[0][s];
          if (GLU) v = glu_apply(y[0][s], y[1][s], alpha, beta, limit);
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
  if (glu && N % 2 != 0) return MOE_ERR_ALIGN;
  if (act_per_slot != 0 && act_per_slot != 1) return MOE_ERR_UNSUPPORTED;
  const size_t lds = (size_t)kGemvSlotBatch * K * sizeof(float);
  if (lds > 64 * 1024) return MOE_ERR_SHAPE;  // K <= 4096
  if (T == 0) return MOE_OK;
  if (!act || !topk_ids || !w || !w_scale || !out) return MOE_ERR_NULL;
  const int n_out = glu ? N / 2 : N;
  dim3 grid((n_out + kGemvColsPerBlock - 1) / kGemvColsPerBlock, T * k);
  hipStream_t st = (hipStream_t)stream;
#define MOE_GEMV_LAUNCH(MX, G)                                                               \
  hipLaunchKernelGGL((sparse_gemv_kernel<MX, G>), grid, dim3(kGemvThreads), lds, st, act,      \
                     act_per_slot, topk_ids, T, k, expert_start, E_local, N, K, w, w_scale, bias, \
                     glu_alpha, glu_beta, glu_limit, out, slot_row)
  const bool mx = wfmt == MOE_W_MXFP4_G32;
  if (mx && glu) MOE_GEMV_LAUNCH(true, true);
  else if (mx) MOE_GEMV_LAUNCH(true, false);
  else if (glu) MOE_GEMV_LAUNCH(false, true);
  else MOE_GEMV_LAUNCH(false, false);
#undef MOE_GEMV_LAUNCH
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
