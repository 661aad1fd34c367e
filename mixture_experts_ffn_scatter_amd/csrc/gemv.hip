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
// activations of those slots are staged in LDS as bf16. A wave computes
// 4 output columns (4 gate + 4 up rows when the GLU is fused): it issues the
// 16-byte weight chunks of all its rows (strided by the wave over K) before
// any arithmetic, converts each chunk to exact bf16 pairs and accumulates
// bf16 dot products in fp32 against the LDS activations; the 64 partial sums
// of a column are folded by shuffles. With the GLU fused, gate row j and up
// row j + N/2 are computed by the same wave and the GLU is applied to their
// bf16-rounded results before the single bf16 store.
#include <cmath>

#include "common.h"

namespace moe {

constexpr int kGemvThreads = 256;
constexpr int kGemvColsPerWave = 4;   // output columns per wave (GLU: 4 gate + 4 up rows)
constexpr int kGemvColsPerBlock = kGemvColsPerWave * (kGemvThreads / 64);
constexpr int kGemvMaxSlots = 64;     // T*k
constexpr int kGemvSlotBatch = 8;     // slots whose activations are staged in LDS at once
constexpr int kGemvMaxChunks = 4;     // 16-byte weight chunks per lane and row (K <= 4096)

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

template <bool MXFP4, bool GLU>
__global__ __launch_bounds__(kGemvThreads) void sparse_gemv_kernel(
    const uint16_t* __restrict__ act, int act_per_slot, const int32_t* __restrict__ ids, int T,
    int k, int expert_start, int E_local, int N, int K, const uint8_t* __restrict__ W,
    const void* __restrict__ w_scale, const uint16_t* __restrict__ bias, float alpha,
    float beta, float limit, uint16_t* __restrict__ out, int32_t* __restrict__ slot_row) {
  extern __shared__ __attribute__((aligned(16))) uint16_t s_act[];  // [kGemvSlotBatch][K] bf16
  __shared__ int s_slots[kGemvMaxSlots];
  __shared__ int s_nslots;

  const int q = blockIdx.y;  // flattened slot t*k+s
  const int tid = threadIdx.x;
  const int nq = T * k;
  const int id = ids[q];
  const int e = id - expert_start;
  const bool local = e >= 0 && e < E_local;
  if (blockIdx.x == 0 && tid == 0 && slot_row) slot_row[q] = local ? q : -1;
  if (!local) return;  // block-uniform, before any LDS use or barrier
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
  const int kchunk = MXFP4 ? 32 : 16;  // weights per 16-byte chunk
  const int nchunks = K / kchunk;
  const uint8_t* We = W + (size_t)e * N * row_bytes;
  const float fp8_scale = MXFP4 ? 1.f : reinterpret_cast<const float*>(w_scale)[e];
  const uint8_t* Ws = MXFP4 ? reinterpret_cast<const uint8_t*>(w_scale) + (size_t)e * N * (K / 32)
                            : nullptr;
  constexpr int kRows = kGemvColsPerWave;       // weight rows per load batch
  constexpr int kHalves = GLU ? 2 : 1;          // gate rows, then up rows

  for (int sb = 0; sb < nslots; sb += kGemvSlotBatch) {
    const int S = min(kGemvSlotBatch, nslots - sb);
    __syncthreads();
    for (int i = tid; i < S * (K / 8); i += kGemvThreads) {
      const int s = i / (K / 8), c8 = i - s * (K / 8);
      const int p = s_slots[sb + s];
      const int arow = act_per_slot ? p : p / k;
      reinterpret_cast<v4i*>(s_act + (size_t)s * K)[c8] =
          reinterpret_cast<const v4i*>(act + (size_t)arow * K)[c8];
    }
    __syncthreads();

    float y[kHalves][kRows][kGemvSlotBatch];
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf) {
      // issue every chunk of the batch's rows before any arithmetic
      v4i raw[kRows][kGemvMaxChunks];
      float gsc[kRows][kGemvMaxChunks];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int j = min(col0 + r, n_out - 1);
        const int n = j + hf * (N / 2);
        const uint8_t* wr = We + (size_t)n * row_bytes;
#pragma unroll
        for (int c = 0; c < kGemvMaxChunks; ++c) {
          const int ch = lane + 64 * c;
          raw[r][c] = v4i{0, 0, 0, 0};
          gsc[r][c] = 0.f;
          if (ch < nchunks) {
            raw[r][c] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wr + (size_t)ch * 16));
            if (MXFP4) gsc[r][c] = e8m0_value(Ws[(size_t)n * (K / 32) + ch]);
          }
        }
      }
      float acc[kRows][kGemvSlotBatch];
#pragma unroll
      for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int s = 0; s < kGemvSlotBatch; ++s) acc[r][s] = 0.f;
#pragma unroll
      for (int c = 0; c < kGemvMaxChunks; ++c) {
        const int ch = lane + 64 * c;
        if (ch >= nchunks) break;
        const int kb = ch * kchunk;
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
          v2bf wp[16];
          weights_to_bf16<MXFP4>(raw[r][c], wp);
#pragma unroll
          for (int s = 0; s < kGemvSlotBatch; ++s) {
            if (s < S) {
              const v2bf* ap = reinterpret_cast<const v2bf*>(s_act + (size_t)s * K + kb);
              float part = 0.f;
#pragma unroll
              for (int i = 0; i < (MXFP4 ? 16 : 8); ++i)
                part = __builtin_amdgcn_fdot2_f32_bf16(wp[i], ap[i], part, false);
              acc[r][s] = MXFP4 ? fmaf(part, gsc[r][c], acc[r][s]) : acc[r][s] + part;
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int j = min(col0 + r, n_out - 1);
        const int n = j + hf * (N / 2);
        const float bv = bias ? bf16_to_f32(bias[(size_t)e * N + n]) : 0.f;
#pragma unroll
        for (int s = 0; s < kGemvSlotBatch; ++s) {
          if (s < S) {
            const float tot = wave_sum_f32(acc[r][s]);
            const float yv = MXFP4 ? __fadd_rn(tot, bv) : __fadd_rn(__fmul_rn(tot, fp8_scale), bv);
            y[hf][r][s] = bf16_to_f32((uint16_t)f32_to_bf16_bits(yv));
          }
        }
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int j = col0 + r;
        if (j >= n_out) break;
#pragma unroll
        for (int s = 0; s < kGemvSlotBatch; ++s) {
          if (s >= S) break;
          const int p = s_slots[sb + s];
          float v = y[0][r][s];
          if (GLU) v = glu_apply(y[0][r][s], y[kHalves - 1][r][s], alpha, beta, limit);
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
  if (K / kchunk > 64 * kGemvMaxChunks) return MOE_ERR_SHAPE;  // K <= 4096 (FP8) / 8192 (MXFP4)
  if (lds > 64 * 1024) return MOE_ERR_SHAPE;
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
