"""Pins for oracle/formats.py against routes that share none of its code:
torch's CPU casts (library routines), decimal arithmetic, and the bit-level
definitions of each format written out independently here."""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

from oracle import formats as F


def _torch_bf16(x32):
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch_for_fp32():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    specials = np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, 3.4e38, 1e-40, -1e-45,
                         np.float32(1.0) + np.float32(2**-8), np.float32(1.0) + np.float32(3 * 2**-9)],
                        dtype=np.float32)
    x = np.concatenate([x, specials]).astype(np.float32)
    assert np.array_equal(F.round_to_bf16(x), _torch_bf16(x))


def test_bf16_rounding_fp64_is_nearest_ties_even():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(20_000) * np.exp2(rng.integers(-140, 120, 20_000))
    # exact midpoints between two bf16 values must go to the even pattern
    base = F.bf16_to_f32(rng.integers(0x0080, 0x7F00, 500).astype(np.uint16)).astype(np.float64)
    nxt = np.nextafter(base.astype(np.float32), np.float32(np.inf)).astype(np.float64)
    up = F.bf16_to_f32(F.round_to_bf16(base) + 1).astype(np.float64)
    mids = (base + up) / 2.0
    del nxt
    x = np.concatenate([x, mids])
    b = F.round_to_bf16(x)
    v = F.bf16_to_f32(b).astype(np.float64)
    lo = F.bf16_to_f32(b - 1).astype(np.float64)
    hi = F.bf16_to_f32(b + 1).astype(np.float64)
    pos = x > 0
    for arr_nb in (lo, hi):
        d_self = np.abs(x - v)
        d_nb = np.abs(x - arr_nb)
        assert np.all((d_self < d_nb) | ((d_self == d_nb) & (b % 2 == 0)) | ~pos | ~np.isfinite(arr_nb))
    assert np.all(F.round_to_bf16(mids) % 2 == 0)


def test_e4m3_decode_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    assert np.array_equal(F.E4M3_VALUES, ref, equal_nan=True)
    assert np.isnan(F.E4M3_VALUES[0x7F]) and np.isnan(F.E4M3_VALUES[0xFF])
    assert F.E4M3_VALUES[0x7E] == 448.0 and F.E4M3_VALUES[1] == 2.0 ** -9


def _structured_fp32(max_abs=448.0):
    """All exponents in e4m3's range and below, with every top-4-bit mantissa
    pattern crossed with low-bit patterns that sit on, just below and just
    above each rounding midpoint, plus random bits."""
    rng = np.random.default_rng(3)
    vals = []
    for ex in range(127 - 24, 127 + 9):
        for top in range(16):
            for low in (0, 1, 0x3FFFF, 0x40000, 0x40001, 0x7FFFF, 0x20000, 0x60000):
                bits = (ex << 23) | (top << 19) | low
                vals.append(bits)
            vals.extend(((ex << 23) | (top << 19) | rng.integers(0, 1 << 19, 8)).tolist())
    b = np.array(vals, dtype=np.uint32)
    x = b.view(np.float32)
    x = x[np.abs(x) <= max_abs]
    return np.concatenate([x, -x, rng.uniform(-448, 448, 200_000).astype(np.float32)])


def test_e4m3_rne_matches_torch_in_range():
    x = _structured_fp32()
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_rne_satfinite(x), ref)


def test_e4m3_roundtrip_ties_saturation_signs():
    fin = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(F.e4m3_rne_satfinite(F.E4M3_VALUES[fin].astype(np.float32)), fin)
    # every midpoint between neighbours goes to the even code
    pos = F.E4M3_VALUES[:127]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.all((pos[:-1] + pos[1:]) / 2 == mids)   # midpoints are exact in fp32
    got = F.e4m3_rne_satfinite(mids)
    assert np.all(got % 2 == 0)
    assert np.all((got == np.arange(126)) | (got == np.arange(1, 127)))
    big = np.array([448.0, 449.0, 480.0, 1e30, np.inf, -1e30, -np.inf], np.float32)
    assert F.e4m3_rne_satfinite(big).tolist() == [0x7E] * 5 + [0xFE] * 2
    assert F.e4m3_rne_satfinite(np.array([np.nan], np.float32))[0] == 0x7F
    assert F.e4m3_rne_satfinite(np.array([-0.0, 0.0], np.float32)).tolist() == [0x80, 0x00]


def test_e2m1_table_matches_bit_formula():
    for c in range(16):
        sign = -1.0 if c & 8 else 1.0
        ex = (c >> 1) & 3
        m = c & 1
        mag = m * 0.5 if ex == 0 else (1.0 + m / 2.0) * 2.0 ** (ex - 1)
        assert F.E2M1_VALUES[c] == sign * mag and math.copysign(1, F.E2M1_VALUES[c]) == sign


def test_e2m1_unpack_low_nibble_first():
    packed = np.array([[0x21, 0xF7]], np.uint8)
    assert F.e2m1_unpack(packed).tolist() == [[1, 2, 7, 15]]


def test_e8m0_decode_matches_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float32).numpy().astype(np.float64)
    got = F.e8m0_decode(np.arange(256))
    assert np.array_equal(got, ref, equal_nan=True)
    assert np.isnan(got[255]) and got[127] == 1.0 and got[0] == 2.0 ** -127


def _ceil_pow2_byte(q: float) -> int:
    """Smallest j >= -127 with 2^j >= q, as a byte j+127 (0 for q == 0)."""
    if q == 0.0:
        return 0
    m, e = math.frexp(q)          # q = m * 2^e, 0.5 <= m < 1
    j = e - 1 if m == 0.5 else e
    return max(j, -127) + 127


def test_ue8m0_rule_equals_ceil_power_of_two():
    rng = np.random.default_rng(4)
    vals = []
    for ex in range(0, 0xF7):
        for m in (0, 1, 0x3FFFFF, 0x400000, 0x400001, 0x7FFFFF):
            vals.append((ex << 23) | m)
        vals.extend(((ex << 23) | rng.integers(0, 1 << 23, 20)).tolist())
    q = np.array(vals, dtype=np.uint32).view(np.float32)
    got = F.ue8m0_ceil_byte(q)
    want = np.array([_ceil_pow2_byte(float(v)) for v in q], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_quant_mx_matches_torch_cast_with_ceil_scale():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    v[3, :32] = 0.0
    v[4, 32:64] = 7.25
    codes, b = F.quant_mx_e4m3(v)
    g = v.reshape(64, 8, 32).astype(np.float64)
    amax = np.abs(g).max(-1)
    want_b = np.array([[_ceil_pow2_byte(float(np.float32(np.float32(a) / np.float32(448.0))))
                        for a in row] for row in amax], np.uint8)
    assert np.array_equal(b, want_b)
    sf = np.exp2(want_b.astype(np.float64) - 127)
    y = (g / sf[..., None]).astype(np.float32).reshape(64, 256)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    # properties: the scale bounds the group, the payload never saturates
    assert np.all(sf >= amax / 448.0)
    assert np.all(np.abs(F.e4m3_decode(codes)) <= 448.0)
    assert b[3, 0] == 0 and set(codes[3, :32].tolist()) <= {0x00}
    # a constant group: v/sf lies in (224, 448], so every code decodes to the
    # same value in [224, 448] (RNE may land on 224 itself)
    cv = F.e4m3_decode(codes[4, 32:64])
    assert np.all(cv == cv[0]) and 224.0 <= cv[0] <= 448.0


def test_pack_words_little_endian():
    b = np.array([[1, 2, 3, 4, 250, 251, 252, 253]], np.uint8)
    w = F.pack_ue8m0_words(b)
    assert w.view(np.uint32)[0, 0] == int.from_bytes(bytes([1, 2, 3, 4]), "little")
    assert w.view(np.uint32)[0, 1] == int.from_bytes(bytes([250, 251, 252, 253]), "little")
    assert np.array_equal(F.unpack_ue8m0_words(w), b)


def _decimal_f32(d: Decimal) -> np.float32:
    # independent nearest-fp32 search: scan a window of candidates by exact distance
    c = np.float32(float(d))
    cands = [c]
    for _ in range(2):
        cands.append(np.nextafter(cands[-1], np.float32(np.inf)))
    lo = c
    for _ in range(2):
        lo = np.nextafter(lo, np.float32(-np.inf))
        cands.append(lo)
    best = min(cands, key=lambda z: (abs(Decimal(float(z)) - d),
                                     int(np.float32(z).view(np.uint32)) & 1))
    return np.float32(best)


def _sigmoid_decimal(v: float) -> Decimal:
    d = Decimal(v)
    if d >= 0:
        return Decimal(1) / (Decimal(1) + (-d).exp())
    e = d.exp()
    return e / (Decimal(1) + e)


def test_sigmoid_correctly_rounded_on_every_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = F.bf16_to_f32(bits)
    x = x[np.isfinite(x)]
    got = F.sigmoid_f32(x)
    getcontext().prec = 50
    want = np.array([_decimal_f32(_sigmoid_decimal(float(v))) for v in x], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_sigmoid_correctly_rounded_random_fp32():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(3000) * 8).astype(np.float32)
    got = F.sigmoid_f32(x)
    getcontext().prec = 50
    want = np.array([_decimal_f32(_sigmoid_decimal(float(v))) for v in x], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
