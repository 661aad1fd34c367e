"""Pins for the MX GEMM and the activation quantiser of oracle/moe.py.

The GEMM is checked against a pure-Python loop that decodes every byte and
nibble from the format bit layouts (written independently here) and sums
with exact rational arithmetic; plus one-hot rows and scale doubling. The
activation is checked against scipy's expit in fp64 and special cases."""
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

from oracle import formats as F
from oracle import moe as M


def _e4m3_bits(c):
    s = -1 if c & 0x80 else 1
    e, m = (c >> 3) & 15, c & 7
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 64)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def _e2m1_bits(c):
    s = -1 if c & 8 else 1
    e, m = (c >> 1) & 3, c & 1
    if e == 0:
        return s * Fraction(m, 2)
    return s * (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)


def _pow2(b):
    return Fraction(2) ** (int(b) - 127)


def _loop_gemm(aq, ab, wp, wb):
    R, K = aq.shape
    N = wp.shape[0]
    out = [[Fraction(0)] * N for _ in range(R)]
    for r in range(R):
        for n in range(N):
            acc = Fraction(0)
            for kk in range(K):
                byte = int(wp[n, kk // 2])
                nib = byte & 0xF if kk % 2 == 0 else byte >> 4
                a = _e4m3_bits(int(aq[r, kk])) * _pow2(ab[r, kk // 32])
                w = _e2m1_bits(nib) * _pow2(wb[n, kk // 32])
                acc += a * w
            out[r][n] = acc
    return out


def _rand_codes_e4m3(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3A        # no NaN codes
    return c


def test_mx_gemm_equals_exact_rational_loop():
    rng = np.random.default_rng(11)
    R, N, K = 3, 5, 96
    aq = _rand_codes_e4m3(rng, (R, K))
    ab = rng.integers(118, 130, size=(R, K // 32)).astype(np.uint8)
    wp = rng.integers(0, 256, size=(N, K // 2)).astype(np.uint8)
    wb = rng.integers(123, 128, size=(N, K // 32)).astype(np.uint8)
    out, exact, tsum = M.mx_gemm(aq, ab, wp, wb)
    ref = _loop_gemm(aq, ab, wp, wb)
    for r in range(R):
        for n in range(N):
            assert Fraction(float(exact[r, n])) == ref[r][n]
    assert np.array_equal(out, F.round_to_bf16(exact))


def test_mx_gemm_one_hot_and_scale_doubling():
    rng = np.random.default_rng(12)
    R, N, K = 4, 6, 128
    aq = _rand_codes_e4m3(rng, (R, K))
    ab = rng.integers(120, 130, size=(R, K // 32)).astype(np.uint8)
    # weight row n is 1.0 (e2m1 code 2) at column 7n+1 and 0 elsewhere, scale 1.0
    wp = np.zeros((N, K // 2), np.uint8)
    wb = np.full((N, K // 32), 127, np.uint8)
    for n in range(N):
        col = 7 * n + 1
        wp[n, col // 2] = 2 << (4 * (col % 2))
    out, exact, _ = M.mx_gemm(aq, ab, wp, wb)
    A = M.dequant_e4m3_rows(aq, ab)
    for n in range(N):
        assert np.array_equal(exact[:, n], A[:, 7 * n + 1])
    # raising one weight group's scale byte by one doubles that group's share
    wp2 = rng.integers(0, 256, size=(N, K // 2)).astype(np.uint8)
    wb2 = rng.integers(123, 127, size=(N, K // 32)).astype(np.uint8)
    _, base, _ = M.mx_gemm(aq, ab, wp2, wb2)
    wb3 = wb2.copy()
    wb3[:, 2] += 1
    _, bumped, _ = M.mx_gemm(aq, ab, wp2, wb3)
    W = M.dequant_mxfp4_rows(wp2, wb2)
    share = A[:, 64:96] @ W[:, 64:96].T
    assert np.array_equal(bumped - base, share)


def test_mx_gemm_exactness_guard_fires():
    aq = np.array([[0x7E, 0x01] + [0] * 30], np.uint8)          # 448 and 2^-9
    ab = np.array([[254]], np.uint8)
    wp = np.array([[0x22] + [0] * 15], np.uint8)
    wb = np.array([[0]], np.uint8)
    # both terms share a group; the span is small, so this is exact
    M.mx_gemm(aq, ab, wp, wb)
    # two groups with scales 2^-127 and 2^127 cannot be summed exactly in fp64
    aq2 = np.array([[0x7E] + [0] * 31 + [0x01] + [0] * 31], np.uint8)
    ab2 = np.array([[254, 0]], np.uint8)
    wp2 = np.full((1, 32), 0x22, np.uint8)
    wb2 = np.array([[127, 127]], np.uint8)
    with pytest.raises(AssertionError):
        M.mx_gemm(aq2, ab2, wp2, wb2)


def test_act_matches_fp64_formula_within_roundings():
    rng = np.random.default_rng(13)
    I = 256
    gu = F.round_to_bf16(rng.standard_normal((16, 2 * I)) * 3)
    h = M.act_rows_f32(gu, I).astype(np.float64)
    g = F.bf16_to_f32(gu[:, :I]).astype(np.float64)
    u = F.bf16_to_f32(gu[:, I:]).astype(np.float64)
    ref = g * expit(g) * u
    # sigma rounded once, two products rounded once each: < 2 ulp of fp32
    assert np.all(np.abs(h - ref) <= 2.0 ** -22 * np.abs(ref) + 1e-44)


def test_act_special_cases_and_clamp():
    I = 128
    def row(g, u):
        gu = np.zeros((1, 2 * I), np.float32)
        gu[0, :I] = g
        gu[0, I:] = u
        return F.round_to_bf16(gu)
    assert np.all(M.act_rows_f32(row(0.0, 5.0), I) == 0)
    assert np.all(M.act_rows_f32(row(3.0, 0.0), I) == 0)
    assert np.all(M.act_rows_f32(row(200.0, 2.0), I) == 400.0)          # sigma(200) == 1.0f
    assert np.all(M.act_rows_f32(row(-200.0, 2.0), I) == 0.0)           # sigma(-200) == 0.0f
    L = 25.0
    assert np.array_equal(M.act_rows_f32(row(40.0, 1.0), I, L), M.act_rows_f32(row(25.0, 1.0), I, L))
    assert np.array_equal(M.act_rows_f32(row(1.0, -90.0), I, L), M.act_rows_f32(row(1.0, -25.0), I, L))
    assert np.array_equal(M.act_rows_f32(row(-90.0, 3.0), I, L), M.act_rows_f32(row(-90.0, 3.0), I))
    # an all-zero group gives scale byte 0 and +-0 codes
    q, b = M.act_quant_rows(row(0.0, 1.0), I)
    assert np.all(b == 0) and set(np.unique(q).tolist()) <= {0x00, 0x80}


def test_act_quant_codes_reconstruct_activation():
    rng = np.random.default_rng(14)
    I = 512
    gu = F.round_to_bf16(rng.standard_normal((8, 2 * I)))
    h = M.act_rows_f32(gu, I).astype(np.float64)
    q, b = M.act_quant_rows(gu, I)
    rec = M.dequant_e4m3_rows(q, b)
    sf = np.repeat(F.e8m0_decode(b), 32, axis=-1)
    # e4m3 keeps 3 mantissa bits: error <= 2^-4 relative, or half the
    # smallest subnormal step (2^-10 * sf) for tiny values
    assert np.all(np.abs(rec - h) <= np.maximum(2.0 ** -4 * np.abs(h), 2.0 ** -10 * sf))
