// Device helpers shared by the gfx950 kernels of the MoE FFN library.
//
// Number formats (OCP MX / FP8 definitions): bf16 = upper half of an fp32;
// E4M3 ("E4M3FN": bias 7, 3 mantissa bits, max 448, no infinities); E2M1
// (bias 1, 1 mantissa bit, magnitudes 0..6); E8M0 (value 2^(b-127)).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_ffn.h"

namespace moe {

constexpr int kWave = 64;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round-to-nearest-even fp32 -> bf16; NaN becomes a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// both to bf16 with one hardware conversion (round to nearest even; NaN
// handling is left to the caller): lo in the low half
typedef __bf16 moe_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float moe_f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne_bits(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((moe_f32x2_t){lo, hi}, moe_bf16x2_t));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------- E8M0 / FP8

// UE8M0 round-up of a non-negative fp32 scale: the fp32 exponent field,
// plus one when the mantissa is non-zero and the exponent is not 0xFE,
// except for subnormals whose mantissa is <= 0x400000; low 8 bits.
__device__ __forceinline__ uint32_t ue8m0_ceil_byte(float q) {
  uint32_t bits = __float_as_uint(q);
  uint32_t ex = bits >> 23;
  uint32_t m = bits & 0x7FFFFFu;
  bool up = (m != 0u) && (ex != 0xFEu) && !(ex == 0u && m <= 0x400000u);
  return (ex + (up ? 1u : 0u)) & 0xFFu;
}

// The same byte for q = fl32(amax / 448), taken from amax's own bits when
// the quotient is normal (amax's exponent field >= 10). With amax = 1.m *
// 2^(ex-127), amax/448 = (1.m/1.75) * 2^(ex-135): the power of two at or
// above it is 2^(ex-135) when 1.m <= 1.75 (mantissa field <= 0x600000),
// else 2^(ex-134). Rounding a normal quotient to fp32 never moves it onto a
// power of two from above (448 * 2^j is an fp32 value and its neighbours
// are more than half an ulp of the quotient away), so the exact quotient
// decides. A subnormal quotient can round onto 2^-127 from above, so
// smaller amax takes the division. Infinity gives 0xFF and NaN 0x00, as the
// rule gives for inf/448 and NaN/448.
__device__ __forceinline__ uint32_t ue8m0_byte_of_amax(float amax) {
  const uint32_t bits = __float_as_uint(amax);
  const int ex = (int)((bits >> 23) & 0xFFu);
  const uint32_t m = bits & 0x7FFFFFu;
  if (ex < 10) return ue8m0_ceil_byte(amax / 448.0f);
  if (ex == 0xFF) return m == 0u ? 0xFFu : 0x00u;
  return (uint32_t)(ex - 8) + (m > 0x600000u ? 1u : 0u);
}

// 2^(127-b) as an fp32, exactly (b <= 254): the reciprocal of the E8M0
// scale 2^(b-127). Multiplying by it equals dividing by the scale, since
// both are one correctly rounded operation on the same real value.
__device__ __forceinline__ float e8m0_reciprocal(uint32_t b) {
  b = b > 254u ? 254u : b;
  return __uint_as_float(b == 254u ? 0x00400000u : (254u - b) << 23);
}

__device__ __forceinline__ float e8m0_value(uint32_t b) {
  // 2^(b-127); b == 0 is the subnormal 2^-127, b == 255 (NaN) is not produced here
  return __uint_as_float(b == 0u ? 0x00400000u : (b << 23));
}

// Two fp32 -> two E4M3 codes, round to nearest even, into the low or high
// 16 bits of `old` (gfx950 OCP FP8 conversion).
template <bool HI>
__device__ __forceinline__ uint32_t cvt_e4m3x2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// ------------------------------------------------------------ reductions

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// ------------------------------------------------------------ layout

__device__ __forceinline__ int align_up_dev(int x, int a) { return ((x + a - 1) / a) * a; }

// Start and end of local expert e in the grouped layout, rebuilt from the
// stored ends: start_0 = 0, start_e = align_up(end_{e-1}, A). Values are
// clamped to [0, M_cap] so that corrupt metadata cannot leave the buffers.
__device__ __forceinline__ void expert_range(const int32_t* __restrict__ ends, int e, int A,
                                             int M_cap, int& start, int& end) {
  int prev = e == 0 ? 0 : ends[e - 1];
  prev = min(max(prev, 0), M_cap);
  int s = min(align_up_dev(prev, A), M_cap);
  int en = min(max(ends[e], s), M_cap);
  start = s;
  end = en;
}

// Expert e's live rows in either layout. slab == 0: the aligned layout,
// meta = expert_ends (expert_range above). slab = m_pad > 0: the masked slab
// layout, meta = masked_m; expert e owns rows [e*m_pad, (e+1)*m_pad) and
// its live rows are the first masked_m[e] of them (clamped into [0, m_pad]
// so that a corrupt count cannot leave the slab).
__device__ __forceinline__ void layout_range(const int32_t* __restrict__ meta, int e, int A,
                                             int M_cap, int slab, int& start, int& end) {
  if (slab > 0) {
    start = e * slab;
    end = start + min(max(meta[e], 0), slab);
  } else {
    expert_range(meta, e, A, M_cap, start, end);
  }
}

}  // namespace moe

// Host-side launch check shared by the entry points.
#define MOE_CHECK_LAUNCH()                                   \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH; \
  } while (0)
