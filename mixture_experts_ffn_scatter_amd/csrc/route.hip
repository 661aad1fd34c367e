// moe_route: top-k expert selection and routing weights on gfx950.
//
// One 64-lane wave per token. Each lane holds ceil(E/64) scores in
// registers; k rounds of a wave-wide arg-max (key descending, expert index
// ascending on ties) pick the experts, and lane s keeps the winner of round
// s. Softmax weights are the softmax over the selected k ("Blackwell
// DeepGEMM FusedMoE (sglang)", section 1; "Phase 20: Sparse MoE Decode",
// section 1). Sigmoid routing selects on sigmoid(logit) + correction bias and
// weights the unbiased sigmoid, renormalised ("Kimi-K3 on SM120 FlashInfer
// MXFP4", Phase 1 call chain). The sigmoid used for selection is the fp32
// rounding of a fp64 evaluation, i.e. the correctly rounded value except
// where an fp64 result falls within a few fp64 ulps of an fp32 midpoint.
#include "common.h"

namespace moe {

constexpr int kRouteTokensPerBlock = 4;
constexpr int kRouteMaxE = 1024;
constexpr int kRouteMaxK = 32;

struct Cand {
  float key;
  int idx;     // expert id; INT32_MAX marks "no candidate"
  float aux;   // sigmoid value (sigmoid mode) or logit (softmax mode)
};

__device__ __forceinline__ bool better(const Cand& a, const Cand& b) {
  return a.key > b.key || (a.key == b.key && a.idx < b.idx);
}

template <int PER_LANE, bool SIGMOID>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, const float* __restrict__ bias,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRouteTokensPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform
  const float* row = logits + (size_t)t * E;

  float key[PER_LANE];
  float aux[PER_LANE];
#pragma unroll
  for (int j = 0; j < PER_LANE; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      const float v = row[e];
      if (SIGMOID) {
        const double s64 = 1.0 / (1.0 + exp(-(double)v));
        const float s = (float)s64;
        aux[j] = s;
        key[j] = __fadd_rn(s, bias[e]);
      } else {
        aux[j] = v;
        key[j] = v;
      }
    } else {
      key[j] = -__builtin_inff();
      aux[j] = 0.f;
    }
  }

  uint32_t taken = 0;
  int my_id = -1;
  float my_aux = 0.f;
  for (int s = 0; s < k; ++s) {
    Cand best{-__builtin_inff(), INT32_MAX, 0.f};
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) {
      const int e = lane + 64 * j;
      Cand c{key[j], e, aux[j]};
      if (e < E && !((taken >> j) & 1u) && better(c, best)) best = c;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      Cand o{__shfl_xor(best.key, m, 64), __shfl_xor(best.idx, m, 64),
             __shfl_xor(best.aux, m, 64)};
      if (better(o, best)) best = o;
    }
    if (best.idx < E && (best.idx & 63) == lane) taken |= 1u << (best.idx >> 6);
    if (lane == s) {
      my_id = best.idx;
      my_aux = best.aux;
    }
  }

  // weights over the k selected slots, evaluated in fp64 and rounded once
  double num;
  if (SIGMOID) {
    num = (double)my_aux;
  } else {
    const float top = __shfl(my_aux, 0, 64);
    num = exp((double)my_aux - (double)top);
  }
  double v = lane < k ? num : 0.0;
  double sum = v;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    weights[(size_t)t * k + lane] = (float)(num / sum);
  }
}

template <int PER_LANE>
static void launch_route(const float* logits, int T, int E, int k, int score_fn, const float* bias,
                         int32_t* ids, float* weights, hipStream_t st) {
  dim3 grid((T + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock);
  if (score_fn == MOE_SCORE_SIGMOID_BIAS)
    hipLaunchKernelGGL((route_kernel<PER_LANE, true>), grid, dim3(256), 0, st, logits, T, E, k,
                       bias, ids, weights);
  else
    hipLaunchKernelGGL((route_kernel<PER_LANE, false>), grid, dim3(256), 0, st, logits, T, E, k,
                       bias, ids, weights);
}

}  // namespace moe

extern "C" int moe_route(const float* logits, int T, int E, int k, int score_fn,
                         const float* correction_bias, int32_t* topk_ids, float* topk_weights,
                         void* stream) {
  using namespace moe;
  if (T < 0 || E < 1 || E > kRouteMaxE || k < 1 || k > E || k > kRouteMaxK) return MOE_ERR_SHAPE;
  if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID_BIAS)
    return MOE_ERR_UNSUPPORTED;
  if (score_fn == MOE_SCORE_SIGMOID_BIAS && !correction_bias) return MOE_ERR_NULL;
  if (score_fn == MOE_SCORE_SOFTMAX && correction_bias) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights) return MOE_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  const int per_lane = (E + 63) / 64;
  if (per_lane <= 1) launch_route<1>(logits, T, E, k, score_fn, correction_bias, topk_ids, topk_weights, st);
  else if (per_lane <= 2) launch_route<2>(logits, T, E, k, score_fn, correction_bias, topk_ids, topk_weights, st);
  else if (per_lane <= 4) launch_route<4>(logits, T, E, k, score_fn, correction_bias, topk_ids, topk_weights, st);
  else if (per_lane <= 8) launch_route<8>(logits, T, E, k, score_fn, correction_bias, topk_ids, topk_weights, st);
  else launch_route<16>(logits, T, E, k, score_fn, correction_bias, topk_ids, topk_weights, st);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
