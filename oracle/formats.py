"""Number formats used by the MoE path, defined from their specifications.

Test infrastructure only (see the package docstring).

* bf16: the upper 16 bits of an IEEE fp32; rounding is to nearest, ties to
  even, in ONE step from the exact (fp64) value.
* E4M3 (OCP "E4M3FN", torch ``float8_e4m3fn``): sign, 4 exponent bits with
  bias 7, 3 mantissa bits, subnormals m/8 * 2^-6, largest finite 448, the
  all-ones exponent+mantissa pattern is NaN, no infinities. The DeepGEMM
  walkthrough ("Blackwell DeepGEMM FusedMoE (sglang)", section 2.4.1) fixes
  the 448 bound used by the scale rule.
* E2M1 (OCP MX FP4): sign bit 3, 2 exponent bits with bias 1, 1 mantissa
  bit: magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}. Two codes per byte
  ("Kimi-K3 on SM120 FlashInfer MXFP4", checkpoint contract: 1792 = 3584/2);
  which nibble holds which element is not stated there -- the reading used
  here is low nibble = even element.
* E8M0 / UE8M0: an unsigned biased exponent, value 2^(b-127); 0x00..0xFE are
  finite powers of two and 0xFF is NaN ("Kimi-K3 on SM120 FlashInfer
  MXFP4", NaN/Inf decision record).
* The UE8M0 ceiling rule for an fp32 scale follows the bit recipe of
  ``_cast_to_e8m0_with_rounding_up`` described in "Blackwell DeepGEMM
  FusedMoE (sglang)", section 2.3.2 and Appendix A.
"""
from __future__ import annotations

from decimal import Decimal, getcontext

import numpy as np

# --------------------------------------------------------------------- bf16

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x) -> np.ndarray:
    """Exact value (fp32 or fp64 array) -> bf16 bits, one RNE rounding.

    bf16 keeps 8 significant bits and fp32's exponent range: the unit in the
    last place of a normal value in [2^(e-1), 2^e) is 2^(e-8); below 2^-126
    the spacing is fixed at 2^-133. Values that round beyond the largest
    finite bf16 become infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    nan = np.isnan(x)
    _, e = np.frexp(x)
    ulp_exp = np.maximum(e - 8, -133)
    q = np.rint(np.ldexp(x, -ulp_exp))          # numpy rint: ties to even
    y = np.ldexp(q, ulp_exp)
    with np.errstate(over="ignore"):
        y32 = y.astype(np.float32)                   # exact, or +-inf on overflow
    big = np.abs(y) >= 2.0 ** 128
    y32 = np.where(big, np.copysign(np.float32(np.inf), y), y32).astype(np.float32)
    out[...] = (y32.view(np.uint32) >> 16).astype(np.uint16)
    out[nan] = 0x7FC0
    return out


# --------------------------------------------------------------------- E4M3

def _e4m3_table() -> np.ndarray:
    v = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            v[c] = np.nan
        elif e == 0:
            v[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            v[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return v


E4M3_VALUES = _e4m3_table()
E4M3_MAX = 448.0
_E4M3_POS = E4M3_VALUES[:127]       # codes 0x00..0x7E, strictly increasing, 0 .. 448


def e4m3_decode(codes) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_rne_satfinite(x) -> np.ndarray:
    """fp32 value -> E4M3 code: nearest finite code, ties to the even code,
    magnitudes beyond 448 saturate to 448, NaN -> 0x7F, sign kept (-0 -> 0x80).

    Implemented as a search over the 127 non-negative finite values, with no
    bit manipulation, so it can be checked against bit-level converters."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    lo = np.searchsorted(_E4M3_POS, a, side="right") - 1
    lo = np.clip(lo, 0, 126)
    hi = np.minimum(lo + 1, 126)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(take_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 126, code)
    sign = np.signbit(x)
    code = code.astype(np.uint8) | np.where(sign, 0x80, 0).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------- E2M1

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=np.float64)


def e2m1_unpack(packed) -> np.ndarray:
    """u8 [..., K/2] -> codes u8 [..., K]; element 2i is the low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def e2m1_decode(codes) -> np.ndarray:
    return E2M1_VALUES[np.asarray(codes, dtype=np.uint8)]


# --------------------------------------------------------------------- E8M0

def e8m0_decode(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.int64)
    v = np.ldexp(1.0, (b - 127).astype(np.int64))
    return np.where(b == 0xFF, np.nan, v)


def ue8m0_ceil_byte(q) -> np.ndarray:
    """fp32 scale -> UE8M0 byte by the round-up bit rule: take the fp32
    exponent field; add one when the mantissa is non-zero and the exponent
    is not 0xFE, unless the value is subnormal with mantissa <= 0x400000;
    keep the low 8 bits."""
    bits = np.asarray(q, dtype=np.float32).view(np.uint32).astype(np.int64)
    ex = bits >> 23
    m = bits & 0x7FFFFF
    up = (m > 0) & (ex != 0xFE) & ~((ex == 0) & (m <= 0x400000))
    return ((ex + up.astype(np.int64)) & 0xFF).astype(np.uint8)


# ------------------------------------------------------- MX group quantiser

E4M3_MAX_F32 = np.float32(448.0)


def quant_mx_e4m3(v, group: int = 32):
    """Per-group FP8 quantisation with UE8M0 scales (the runtime-activation
    production line of "Blackwell DeepGEMM FusedMoE (sglang)", Appendix A,
    with the ceil-then-divide order of section 2.4.1).

    v: fp32 [..., C] with C % group == 0. For each group of 32:
      amax  = max |v_i|                          (fp32, exact)
      q     = fl32(amax / 448)
      b     = ue8m0_ceil_byte(q)
      sf    = 2^(b-127)
      code_i = e4m3_rne_satfinite(fl32(v_i / sf))
    Returns (codes u8 [..., C], scale bytes u8 [..., C/group]).
    """
    v = np.asarray(v, dtype=np.float32)
    C = v.shape[-1]
    assert C % group == 0
    g = v.reshape(v.shape[:-1] + (C // group, group))
    amax = np.max(np.abs(g), axis=-1)
    q = (amax / E4M3_MAX_F32).astype(np.float32)
    b = ue8m0_ceil_byte(q)
    sf = np.ldexp(np.float32(1.0), b.astype(np.int32) - 127).astype(np.float32)
    with np.errstate(invalid="ignore"):
        y = (g / sf[..., None]).astype(np.float32)
    codes = e4m3_rne_satfinite(y).reshape(v.shape)
    return codes, b


def pack_ue8m0_words(b) -> np.ndarray:
    """u8 [R, G] (G % 4 == 0) -> int32 [R, G/4]; group 4c+j sits in byte j
    of word c (the uint8 -> int32 view of the UE8M0 packing)."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint8))
    R, G = b.shape
    assert G % 4 == 0
    w = (b[:, 0::4].astype(np.uint32) | (b[:, 1::4].astype(np.uint32) << 8)
         | (b[:, 2::4].astype(np.uint32) << 16) | (b[:, 3::4].astype(np.uint32) << 24))
    return w.view(np.int32)


def unpack_ue8m0_words(w) -> np.ndarray:
    w = np.asarray(w, dtype=np.int32).view(np.uint32)
    R, W = w.shape
    b = np.empty((R, W * 4), dtype=np.uint8)
    for j in range(4):
        b[:, j::4] = ((w >> (8 * j)) & 0xFF).astype(np.uint8)
    return b


# ------------------------------------------------------- correctly rounded

def _decimal_to_f32_rne(d: Decimal) -> np.float32:
    """Nearest fp32 to a Decimal, ties to even, by exact comparison."""
    c = np.float32(float(d))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        dist = abs(Decimal(float(cand)) - d)
        key = (dist, int(np.float32(cand).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def sigmoid_exact_decimal(x: float, prec: int = 60) -> Decimal:
    getcontext().prec = prec
    d = Decimal(float(x))
    if d >= 0:
        return Decimal(1) / (Decimal(1) + (-d).exp())
    e = d.exp()                      # e^x for x < 0 never overflows
    return e / (Decimal(1) + e)


def sigmoid_f32(x) -> np.ndarray:
    """Correctly rounded fp32 logistic sigmoid 1/(1+e^-x) of fp32 inputs.

    Evaluated in fp64; where the fp64 value lies too close to an fp32
    rounding midpoint for fp64's error to be ruled out, the value is
    recomputed with 60-digit decimal arithmetic and rounded exactly."""
    x32 = np.asarray(x, dtype=np.float32)
    xd = x32.astype(np.float64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-xd))
    r = s.astype(np.float32)
    lo = np.nextafter(r, np.float32(-np.inf)).astype(np.float64)
    hi = np.nextafter(r, np.float32(np.inf)).astype(np.float64)
    rd = r.astype(np.float64)
    mid_lo = (rd + lo) / 2.0
    mid_hi = (rd + hi) / 2.0
    margin = np.minimum(np.abs(s - mid_lo), np.abs(s - mid_hi))
    bound = 16.0 * np.spacing(np.maximum(np.abs(s), 2.0 ** -1022))
    risky = np.flatnonzero((margin <= bound).ravel() & np.isfinite(xd).ravel())
    out = r.ravel().copy()
    for i in risky:
        out[i] = _decimal_to_f32_rne(sigmoid_exact_decimal(float(x32.ravel()[i])))
    return out.reshape(x32.shape)


def scaled_tanh_exact_decimal(x: float, beta: float, prec: int = 120) -> Decimal:
    """beta * tanh(x / beta) in decimal arithmetic, as (1 - e^(-2y)) /
    (1 + e^(-2y)) for y = |x| / beta (120 digits, so that the cancellation in
    1 - e^(-2y) for the smallest bf16 inputs still leaves far more than
    fp32's precision)."""
    getcontext().prec = prec
    b = Decimal(float(beta))
    y = Decimal(float(x)) / b
    neg = y < 0
    y = -y if neg else y
    e = (-2 * y).exp()               # e^(-2y) <= 1 never overflows
    t = (1 - e) / (1 + e)
    return -(b * t) if neg else b * t


def scaled_tanh_f32(x, beta: float) -> np.ndarray:
    """Correctly rounded fp32 of beta * tanh(x / beta) for fp32 inputs (the
    two factors of the SiTU activation, "DeepGEMM FusedMoE on Blackwell
    (sglang)", section 2.4.1, situ branch: gate factor with beta = 4, up
    factor with beta = 25 for Kimi-K3).

    Evaluated in fp64; where the fp64 value lies too close to an fp32
    rounding midpoint for fp64's error to be ruled out, it is recomputed
    with decimal arithmetic and rounded exactly."""
    x32 = np.asarray(x, dtype=np.float32)
    xd = x32.astype(np.float64)
    s = beta * np.tanh(xd / beta)
    r = s.astype(np.float32)
    lo = np.nextafter(r, np.float32(-np.inf)).astype(np.float64)
    hi = np.nextafter(r, np.float32(np.inf)).astype(np.float64)
    rd = r.astype(np.float64)
    margin = np.minimum(np.abs(s - (rd + lo) / 2.0), np.abs(s - (rd + hi) / 2.0))
    bound = 16.0 * np.spacing(np.maximum(np.abs(s), 2.0 ** -1022))
    risky = np.flatnonzero((margin <= bound).ravel() & np.isfinite(xd).ravel())
    out = r.ravel().copy()
    for i in risky:
        out[i] = _decimal_to_f32_rne(scaled_tanh_exact_decimal(float(x32.ravel()[i]), beta))
    return out.reshape(x32.shape)
