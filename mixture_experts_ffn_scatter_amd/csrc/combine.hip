// moe_combine: unpermute + weighted top-k sum on gfx950.
//
// "Blackwell DeepGEMM FusedMoE (sglang)", section 2.6.1 (post_reorder): per
// token, an fp32 sum over the slots whose destination row is valid of
// weight * row, then times the routed scaling factor, stored as bf16.
// "Phase 20: Sparse MoE Decode", section 3: slots that are not local are
// skipped, never multiplied by zero (their rows may hold NaN garbage).
//
// One block per (token, 2048-column chunk); a lane owns 8 consecutive
// columns (16-byte loads per slot, one 16-byte store). The slot metadata is
// read once per wave (one slot per lane) and the live slots' row loads are
// all issued before the sum, so a token waits for two dependent loads. The sum follows the
// slot order with separately rounded multiply and add, so the result is
// bit-for-bit the fixed fp32 sequence.
#include "common.h"

namespace moe {

constexpr int kCombineMaxK = 32;

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ rows,
                                                      int64_t n_rows,
                                                      const int32_t* __restrict__ row_of_slot,
                                                      const float* __restrict__ weights, int k,
                                                      int H, float scale,
                                                      uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int col = (blockIdx.y * 256 + threadIdx.x) * 8;
  // the token's slots, one per lane, read once; live slots as a wave mask
  int row = -1;
  float wt = 0.f;
  if (lane < k) {
    row = row_of_slot[(size_t)t * k + lane];
    wt = weights[(size_t)t * k + lane];
  }
  const uint64_t live = __ballot(row >= 0 && (int64_t)row < n_rows);
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  const bool in = col < H;
  // live slots in ascending order, up to 8 row loads in flight per lane
  for (uint64_t m = live; m;) {
    uint4 raw[8];
    float w[8];
    int n = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      raw[j] = make_uint4(0, 0, 0, 0);
      w[j] = 0.f;
      if (m) {                                   // wave-uniform
        const int s = __ffsll((unsigned long long)m) - 1;
        m &= m - 1;
        const int r = __builtin_amdgcn_readlane(row, s);
        w[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), s));
        if (in) raw[j] = *reinterpret_cast<const uint4*>(rows + (size_t)r * H + col);
        n = j + 1;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < n) {
        const float v[8] = {bf16_lo(raw[j].x), bf16_hi(raw[j].x), bf16_lo(raw[j].y),
                            bf16_hi(raw[j].y), bf16_lo(raw[j].z), bf16_hi(raw[j].z),
                            bf16_lo(raw[j].w), bf16_hi(raw[j].w)};
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __fadd_rn(acc[i], __fmul_rn(w[j], v[i]));
      }
    }
  }
  if (!in) return;
  uint4 o;
  o.x = pack_bf16x2(__fmul_rn(acc[0], scale), __fmul_rn(acc[1], scale));
  o.y = pack_bf16x2(__fmul_rn(acc[2], scale), __fmul_rn(acc[3], scale));
  o.z = pack_bf16x2(__fmul_rn(acc[4], scale), __fmul_rn(acc[5], scale));
  o.w = pack_bf16x2(__fmul_rn(acc[6], scale), __fmul_rn(acc[7], scale));
  *reinterpret_cast<uint4*>(out + (size_t)t * H + col) = o;
}

}  // namespace moe

extern "C" int moe_combine(const uint16_t* rows, int64_t n_rows, const int32_t* row_of_slot,
                           const float* topk_weights, int T, int k, int H, float routed_scale,
                           uint16_t* out, void* stream) {
  using namespace moe;
  if (T < 0 || k < 1 || k > kCombineMaxK || H <= 0 || n_rows < 0) return MOE_ERR_SHAPE;
  if (H % 8 != 0) return MOE_ERR_ALIGN;
  if (T == 0) return MOE_OK;
  if (!row_of_slot || !topk_weights || !out || (!rows && n_rows > 0)) return MOE_ERR_NULL;
  dim3 grid(T, (H + 2047) / 2048);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, (hipStream_t)stream, rows, n_rows,
                     row_of_slot, topk_weights, k, H, routed_scale, out);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
