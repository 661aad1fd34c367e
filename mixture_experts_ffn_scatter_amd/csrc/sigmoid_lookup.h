// sigma(g) for a bf16-valued g from the generated sigmoid table (include
// sigmoid_table.inc first: it defines the table's exponent range). Entries
// are indexed by sign, exponent field and 7-bit mantissa; exponents outside
// [MOE_SIGMOID_EXP_LO, MOE_SIGMOID_EXP_HI] clamp to the range's ends, whose
// values (0.5, 1 and 0 after rounding) hold for every exponent beyond them.
#pragma once

namespace moe {

__device__ __forceinline__ float sigmoid_lookup_table(const float* tab, float g) {
  const uint32_t bits = __float_as_uint(g) >> 16;  // g is an exact bf16 value
  uint32_t a = bits & 0x7FFFu;
  a = min(max(a, (uint32_t)(MOE_SIGMOID_EXP_LO << 7)), (uint32_t)((MOE_SIGMOID_EXP_HI << 7) | 127));
  const uint32_t idx = a - (MOE_SIGMOID_EXP_LO << 7) +
                       ((bits >> 15) ? (uint32_t)((MOE_SIGMOID_EXP_HI - MOE_SIGMOID_EXP_LO + 1) * 128) : 0u);
  return tab[idx];
}

// The same sigma(g) from a 21 KB subset of the table, for kernels whose LDS
// cannot hold all of it. Rows kept: exponent fields 112..131 of g >= 0 and
// 112..133 of g < 0 (kSigRows of 128). Elsewhere the value follows from the
// table's own structure:
//  - |g| < 2^-15 (field < 112): sigma(g) = 1/2 + g/4 - g^3/48 + ..., and
//    1/2 + g/4 (exact in fp64) lies either on an fp32 rounding tie or at
//    least 2^-34 away from one, while the cubic term is below 2^-50 and
//    pulls toward 1/2; so the value is 1/2 + g/4 rounded to nearest with
//    ties toward 1/2 (a 2^-50 nudge toward 1/2 before the rounding),
//  - g >= 0 with field >= 132 (g >= 32, inf, NaN): 1.0, and g < 0 with
//    field >= 134: 0.0 (the table rows there hold only these values).
// Every bf16 pattern is checked against the full table by a test.
constexpr int kSigPosLo = 112, kSigPosHi = 131, kSigNegLo = 112, kSigNegHi = 133;
constexpr int kSigPosRows = kSigPosHi - kSigPosLo + 1;
constexpr int kSigRows = kSigPosRows + (kSigNegHi - kSigNegLo + 1);

// entry i of the compact table: its index in the full table
__device__ __forceinline__ int sigmoid_compact_source(int i) {
  const int row = i >> 7, m = i & 127;
  if (row < kSigPosRows) return (kSigPosLo - MOE_SIGMOID_EXP_LO + row) * 128 + m;
  return (MOE_SIGMOID_EXP_HI - MOE_SIGMOID_EXP_LO + 1) * 128 +
         (kSigNegLo - MOE_SIGMOID_EXP_LO + row - kSigPosRows) * 128 + m;
}

// The common case as few operations: the kept-row read, with the index
// clamped into the compact table, then the large-|g| constants; values with
// |g| < 2^-15 (rare) are patched by sigmoid_small_fix, which the caller runs
// only when some lane of the wave has one.
__device__ __forceinline__ float sigmoid_lookup_compact_fast(const float* ct, float g) {
  const uint32_t bits = __float_as_uint(g) >> 16;  // g is an exact bf16 value
  const uint32_t neg = bits >> 15;
  const int a = (int)(bits & 0x7FFFu) - kSigPosLo * 128;          // row-major offset
  const int top = neg ? (kSigNegHi - kSigNegLo + 1) * 128 - 1 : kSigPosRows * 128 - 1;
  const int idx = min(max(a, 0), top) + (neg ? kSigPosRows * 128 : 0);
  const float tv = ct[idx];
  return a > top ? (neg ? 0.0f : 1.0f) : tv;
}
__device__ __forceinline__ bool sigmoid_is_small(float g) {
  return ((__float_as_uint(g) >> 23) & 0xFFu) < (uint32_t)kSigPosLo;
}
__device__ __forceinline__ float sigmoid_small_fix(float g, float v) {
  const bool neg = __float_as_uint(g) >> 31;
  const float sv = (float)(0.5 + (double)(g * 0.25f) + (neg ? 0x1p-50 : -0x1p-50));
  return sigmoid_is_small(g) ? sv : v;
}

}  // namespace moe
