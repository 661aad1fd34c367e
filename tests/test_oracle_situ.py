"""Pins for the SiTU activation of oracle/moe.py and its scaled-tanh step
(oracle/formats.py): the fp64 fast path against 120-digit decimal
evaluation of beta * tanh(x / beta), the function's closed-form properties
over every finite bf16 input, and the activation's special cases and its
agreement with an fp64 evaluation of the formula."""
import numpy as np
import pytest

from oracle import formats as F
from oracle import moe as M


def _all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32)
    keep = ((b >> 7) & 0xFF) != 0xFF
    return F.bf16_to_f32(b[keep].astype(np.uint16)).astype(np.float32)


@pytest.mark.parametrize("beta", [4.0, 25.0])
def test_scaled_tanh_equals_decimal_definition(beta):
    """Every 23rd finite bf16 value (about 2,800, all binades) plus values
    around the saturation and identity edges: the correctly rounded fp32 of
    beta * tanh(x / beta), computed exactly in decimal arithmetic."""
    x = _all_finite_bf16()[::23]
    edges = np.array([2.0 ** -12, 2.0 ** -9, 0.5, 1.0, beta, 9 * beta, 10 * beta, 3.0e38],
                     np.float32)
    x = np.concatenate([x, edges, -edges])
    got = F.scaled_tanh_f32(x, beta)
    want = np.array([F._decimal_to_f32_rne(F.scaled_tanh_exact_decimal(float(v), beta)) for v in x],
                    np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("beta", [4.0, 25.0])
def test_scaled_tanh_properties_every_bf16(beta):
    x = _all_finite_bf16()
    f = F.scaled_tanh_f32(x, beta)
    # odd (sign of zero kept), bounded by beta, monotone
    assert np.array_equal(F.scaled_tanh_f32(-x, beta).view(np.uint32), (-f).view(np.uint32))
    assert np.all(np.abs(f) <= beta)
    order = np.argsort(x, kind="stable")
    assert np.all(np.diff(f[order].astype(np.float64)) >= 0)
    # near zero the value is x itself: x - x^3/(3 beta^2) rounds back to x
    small = np.abs(x) <= 2.0 ** -12
    assert np.array_equal(f[small], x[small])
    # far out it saturates at +-beta: beta (1 - tanh(y)) ~ 2 beta e^(-2y) is
    # under half an ulp below beta once y >= 10 (y = 9 is not enough)
    big = np.abs(x) >= 10 * beta
    assert np.array_equal(f[big], np.sign(x[big]) * np.float32(beta))


def test_situ_special_cases():
    I = 32
    def row(g, u):
        return F.round_to_bf16(np.concatenate([np.full(I, g), np.full(I, u)]))[None, :]
    # gate 0 or up 0: exactly zero
    assert np.all(M.act_rows_f32_situ(row(0.0, 3.0), I) == 0)
    assert np.all(M.act_rows_f32_situ(row(2.0, 0.0), I) == 0)
    # large gate: 4 tanh(g/4) = 4 and sigmoid(g) = 1, so h = fl32(4 * 25 tanh(u/25))
    u = np.float32(F.bf16_to_f32(F.round_to_bf16(np.array([7.5]))[0]))
    h = M.act_rows_f32_situ(row(60.0, 7.5), I)
    assert np.all(h == np.float32(4.0) * F.scaled_tanh_f32(np.array([u]), 25.0)[0])
    # large up: the up factor saturates at 25
    h = M.act_rows_f32_situ(row(1.0, 400.0), I)
    a = (F.scaled_tanh_f32(np.array([1.0], np.float32), 4.0) *
         F.sigmoid_f32(np.array([1.0], np.float32))).astype(np.float32)
    assert np.all(h == (a * np.float32(25.0)).astype(np.float32))
    # odd in u, and sign-symmetric structure in g: h(g, -u) = -h(g, u)
    rng = np.random.default_rng(5)
    gu = F.round_to_bf16(rng.standard_normal((4, 2 * I)) * 3)
    neg = gu.copy()
    neg[:, I:] ^= 0x8000
    assert np.array_equal(M.act_rows_f32_situ(neg, I), -M.act_rows_f32_situ(gu, I))


def test_situ_matches_fp64_formula_within_roundings():
    """Five fp32 roundings (three function values, two products) stay within
    a few ulps of the fp64 formula."""
    rng = np.random.default_rng(11)
    I = 256
    gu = F.round_to_bf16(rng.standard_normal((64, 2 * I)) * 4)
    h = M.act_rows_f32_situ(gu, I).astype(np.float64)
    v = F.bf16_to_f32(gu).astype(np.float64)
    g, u = v[:, :I], v[:, I:]
    ref = (4 * np.tanh(g / 4) / (1 + np.exp(-g))) * (25 * np.tanh(u / 25))
    assert np.all(np.abs(h - ref) <= 4 * 2.0 ** -24 * np.abs(ref) + 1e-38)


def test_situ_quant_uses_the_silu_quantiser():
    rng = np.random.default_rng(12)
    I = 128
    gu = F.round_to_bf16(rng.standard_normal((8, 2 * I)) * 2)
    q, b = M.act_quant_rows_situ(gu, I)
    q2, b2 = F.quant_mx_e4m3(M.act_rows_f32_situ(gu, I), 32)
    assert np.array_equal(q, q2) and np.array_equal(b, b2)
