// moe_route: top-k expert selection and routing weights on gfx950.
//
// One 64-lane wave per token. Each lane holds ceil(E/64) scores in
// registers; k rounds of a wave-wide arg-max (key descending, expert index
// ascending on ties) pick the experts, and lane s keeps the winner of round
// s. Softmax weights are the softmax over the selected k ("Blackwell
// DeepGEMM FusedMoE (sglang)", section 1; "Phase 20: Sparse MoE Decode",
// section 1). Sigmoid routing selects on sigmoid(logit) + correction bias and
// weights the unbiased sigmoid, renormalised ("Kimi-K3 on SM120 FlashInfer
// MXFP4", Phase 1 call chain). The sigmoid used for selection is the
// correctly rounded fp32 value of 1/(1+e^-x): an fp64 evaluation decides it
// unless it lies within 2^-47 (relative) of an fp32 rounding midpoint, and
// there a double-double evaluation decides.
#include "common.h"

namespace moe {

// ---------------------------------------------- correctly rounded sigmoid
//
// Double-double arithmetic (a value is hi + lo with |lo| <= ulp(hi)/2):
// the error-free sum of Knuth and the error-free product by fused
// multiply-add, and the usual dd add / multiply / divide built on them.
// (The library compiles with floating-point contraction off, so no
// expression below is fused behind its back.)
struct dd {
  double hi, lo;
};
__device__ __forceinline__ dd dd_two_sum(double a, double b) {
  const double s = a + b;
  const double bb = s - a;
  return {s, (a - (s - bb)) + (b - bb)};
}
__device__ __forceinline__ dd dd_fast_two_sum(double a, double b) {   // |a| >= |b|
  const double s = a + b;
  return {s, b - (s - a)};
}
__device__ __forceinline__ dd dd_add(dd a, dd b) {
  dd s = dd_two_sum(a.hi, b.hi);
  const dd t = dd_two_sum(a.lo, b.lo);
  s.lo += t.hi;
  s = dd_fast_two_sum(s.hi, s.lo);
  s.lo += t.lo;
  return dd_fast_two_sum(s.hi, s.lo);
}
__device__ __forceinline__ dd dd_mul(dd a, dd b) {
  const double p = a.hi * b.hi;
  double e = __builtin_fma(a.hi, b.hi, -p);
  e += a.hi * b.lo + a.lo * b.hi;
  return dd_fast_two_sum(p, e);
}
__device__ __forceinline__ dd dd_mul_d(dd a, double b) {
  const double p = a.hi * b;
  double e = __builtin_fma(a.hi, b, -p);
  e += a.lo * b;
  return dd_fast_two_sum(p, e);
}
// a / b by long division: three quotient digits
__device__ __forceinline__ dd dd_div(dd a, dd b) {
  const double q1 = a.hi / b.hi;
  dd r = dd_add(a, dd_mul_d(b, -q1));
  const double q2 = r.hi / b.hi;
  r = dd_add(r, dd_mul_d(b, -q2));
  const double q3 = r.hi / b.hi;
  return dd_add(dd_fast_two_sum(q1, q2), dd{q3, 0.0});
}

// e^x in double-double for |x| <= 110: x = n ln2 + r with |r| <= ln2/2
// (ln2 as a double-double), e^(r/1024) - 1 by its Taylor series through
// degree 9 (Horner; the first dropped term is below 2^-120 of the sum),
// then ten squarings of 1 + t in the form t <- t (t + 2), and the power of
// two. Relative error well below 2^-90.
__device__ dd dd_exp(double x) {
  const dd ln2{0x1.62e42fefa39efp-1, 0x1.abc9e3b39803fp-56};
  const double n = __builtin_rint(x * 0x1.71547652b82fep0);   // nearest integer to x / ln2
  dd r = dd_add(dd{x, 0.0}, dd_mul_d(ln2, -n));
  r.hi = __builtin_ldexp(r.hi, -10);
  r.lo = __builtin_ldexp(r.lo, -10);
  // 1/j! as a double-double (j! is exact in fp64 for j <= 9)
  auto inv_fact = [](int j) {
    double f = 1.0;
    for (int i = 2; i <= j; ++i) f *= (double)i;
    return dd_div(dd{1.0, 0.0}, dd{f, 0.0});
  };
  // p = 1/1! + r/2! + r^2/3! + ... + r^8/9!
  dd p = inv_fact(9);
  for (int j = 8; j >= 1; --j) p = dd_add(inv_fact(j), dd_mul(r, p));
  dd t = dd_mul(r, p);                                         // e^(r/1024) - 1
  for (int i = 0; i < 10; ++i) t = dd_mul(t, dd_add(t, dd{2.0, 0.0}));
  const dd e = dd_add(dd{1.0, 0.0}, t);
  const int ni = (int)n;
  return {__builtin_ldexp(e.hi, ni), __builtin_ldexp(e.lo, ni)};
}

// neighbours of a non-negative finite fp32 value
__device__ __forceinline__ float f32_up(float f) { return __uint_as_float(__float_as_uint(f) + 1u); }
__device__ __forceinline__ float f32_down(float f) {
  return f > 0.f ? __uint_as_float(__float_as_uint(f) - 1u) : -__uint_as_float(1u);
}

// The fp32 value nearest 1/(1+e^-v), ties to even.
__device__ float sigmoid_f32_rn(float v) {
  const double x = (double)v;
  const double s64 = 1.0 / (1.0 + exp(-x));
  const float f = (float)s64;                 // in [0, 1]
  // the two rounding midpoints around f (exact in fp64, also for subnormal f)
  const double fd = (double)f;
  const double m_lo = 0.5 * (fd + (double)f32_down(f));
  const double m_hi = 0.5 * (fd + (double)f32_up(f));
  const double tol = 0x1p-47 * s64;
  const bool near_lo = __builtin_fabs(s64 - m_lo) <= tol;
  const bool near_hi = __builtin_fabs(s64 - m_hi) <= tol;
  if (!(near_lo || near_hi)) return f;
  if (!(x > -110.0 && x < 110.0)) return f;   // beyond: never near a midpoint
  // double-double: for v >= 0, 1 / (1 + e^-v); for v < 0, e^v / (1 + e^v)
  dd sig;
  if (x >= 0.0) {
    const dd e = dd_exp(-x);
    sig = dd_div(dd{1.0, 0.0}, dd_add(dd{1.0, 0.0}, e));
  } else {
    const dd e = dd_exp(x);
    sig = dd_div(e, dd_add(dd{1.0, 0.0}, e));
  }
  // which side of the midpoint: sig.hi - m is exact near m (Sterbenz)
  const double m = near_hi ? m_hi : m_lo;
  const double side = (sig.hi - m) + sig.lo;
  const bool odd = (__float_as_uint(f) & 1u) != 0;
  if (near_hi) return (side > 0.0 || (side == 0.0 && odd)) ? f32_up(f) : f;
  return (side < 0.0 || (side == 0.0 && odd)) ? f32_down(f) : f;
}

constexpr int kRouteTokensPerBlock = 4;
constexpr int kRouteMaxE = 1024;
constexpr int kRouteMaxK = 32;

// A candidate packed into one integer that orders like (key descending,
// expert index ascending): the key's bits mapped to an unsigned order in the
// high word, the complement of the index in the low word. 0 is below every
// candidate and marks "taken / none".
__device__ __forceinline__ uint64_t pack_cand(float key, int idx) {
  uint32_t b = __float_as_uint(key);
  if (b == 0x80000000u) b = 0;  // -0 ties with +0
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}

// wave-wide maximum with DPP row shifts and row broadcasts (a few cycles per
// step, no LDS traffic); the result of lane 63 is returned to every lane
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, ROWMASK, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, ROWMASK, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp_u64<0x111, 0xF>(v); v = v > o ? v : o;   // row_shr:1
  o = dpp_u64<0x112, 0xF>(v); v = v > o ? v : o;   // row_shr:2
  o = dpp_u64<0x114, 0xF>(v); v = v > o ? v : o;   // row_shr:4
  o = dpp_u64<0x118, 0xF>(v); v = v > o ? v : o;   // row_shr:8
  o = dpp_u64<0x142, 0xA>(v); v = v > o ? v : o;   // row_bcast:15
  o = dpp_u64<0x143, 0xC>(v); v = v > o ? v : o;   // row_bcast:31
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
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
  uint64_t cand[PER_LANE];
  float aux[PER_LANE];
#pragma unroll
  for (int j = 0; j < PER_LANE; ++j) {
    const int e = lane + 64 * j;
    cand[j] = 0;
    aux[j] = 0.f;
    if (e < E) {
      const float v = row[e];
      float key = v;
      if (SIGMOID) {
        aux[j] = sigmoid_f32_rn(v);
        key = __fadd_rn(aux[j], bias[e]);
      } else {
        aux[j] = v;
      }
      cand[j] = pack_cand(key, e);
    }
  }
  // k rounds: the best remaining candidate of the wave; lane s keeps round s
  int my_id = -1;
  float my_aux = 0.f;
  for (int s = 0; s < k; ++s) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) best = cand[j] > best ? cand[j] : best;
    best = wave_max_u64(best);
    const int idx = (int)(0xFFFFFFFFu - (uint32_t)best);   // wave-uniform
    const int owner = idx & 63, slot = idx >> 6;
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j)
      if (j == slot) {
        a = aux[j];
        if (lane == owner) cand[j] = 0;                  // taken
      }
    a = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(a), owner));
    if (lane == s) {
      my_id = idx;
      my_aux = a;
    }
  }
  // weights over the k selected slots, evaluated in fp64 and rounded once;
  // the sum runs in slot order
  double num;
  if (SIGMOID) {
    num = (double)my_aux;
  } else {
    const float top = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_aux), 0));
    num = exp((double)my_aux - (double)top);
  }
  double sum = 0.0;
  for (int s = 0; s < k; ++s) {
    const uint64_t bits = (uint64_t)__double_as_longlong(num);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)bits, s);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(bits >> 32), s);
    sum += __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  }
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
