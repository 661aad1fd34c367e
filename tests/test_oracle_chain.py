"""Pins for the whole-chain formulations of oracle/moe.py: the expert-major
chain (endpoints, permutation, grouped GEMMs, live-row act-quant, combine)
must equal, bit for bit, a token-major chain that has no layout at all;
combine identities; and the sparse decode chain against a dense one."""
import numpy as np

import workloads as W
from oracle import formats as F
from oracle import moe as M


def test_expert_major_equals_token_major_tiny():
    c = W.tiny()
    ids, wts = M.route_softmax(c.logits, c.k)
    r = M.prefill_expert_major(c.x, ids, wts, 0, c.E, c.A, c.I, c.weights.w13, c.weights.s13,
                               c.weights.w2, c.weights.s2)
    tm = M.prefill_token_major(c.x, ids, wts, 0, c.E, c.I, c.weights.w13, c.weights.s13,
                               c.weights.w2, c.weights.s2)
    assert np.array_equal(r.out, tm)
    assert r.scatter.end[-1] <= c.M_cap


def test_expert_major_equals_token_major_window_and_clamp():
    """Local window (experts 2..5 of 8) with -1 slots and a clamp."""
    c = W.tiny(seed=77, T=24)
    ids, wts = M.route_softmax(c.logits, c.k)
    ids = ids.copy()
    ids[3, 1] = -1
    w = c.weights
    r = M.prefill_expert_major(c.x, ids, wts, 2, 4, 16, c.I, w.w13[2:6], w.s13[2:6], w.w2[2:6],
                               w.s2[2:6], clamp=6.0, routed_scale=0.5)
    tm = M.prefill_token_major(c.x, ids, wts, 2, 4, c.I, w.w13[2:6], w.s13[2:6], w.w2[2:6],
                               w.s2[2:6], clamp=6.0, routed_scale=0.5)
    assert np.array_equal(r.out, tm)
    no_local = ~np.any((ids >= 2) & (ids < 6), axis=1)
    assert np.all(r.out[no_local] == 0)


def test_combine_identities():
    rng = np.random.default_rng(15)
    rows = F.bf16_to_f32(F.round_to_bf16(rng.standard_normal((6, 32))))
    # k = 1, weight 1, scale 1 copies the row exactly
    out = M.combine(rows, np.array([4, 1, 5]), np.ones((3, 1), np.float32))
    assert np.array_equal(F.bf16_to_f32(out), rows[[4, 1, 5]])
    # a NaN in a row that only skipped slots would point at never reaches the output
    rows_nan = rows.copy()
    rows_nan[0] = np.nan
    ros = np.array([[1, -1], [-1, 2]])
    w = np.array([[0.5, 0.0], [0.0, 0.25]], np.float32)
    out = M.combine(rows_nan, ros, w)
    assert np.all(np.isfinite(F.bf16_to_f32(out)))
    # all slots skipped -> zero
    assert np.all(M.combine(rows, np.array([[-1, -1]]), np.ones((1, 2), np.float32)) == 0)


def test_decode_sparse_equals_dense_small():
    c = W.decode(T=3, H=64, experts=8, E=8)
    ids, wts = M.route_softmax(c.logits, c.k)
    sp = M.decode_chain(c, ids=ids, weights=wts)
    # dense: every expert on every token, then pick the routed slots
    H = c.H
    dense = {}
    for e in range(c.E):
        g, _ = M.gemv_fp8(c.x, c.w_gu[e], c.s_gu[e], c.b_gu[e])
        a = M.glu(g[:, :H], g[:, H:], c.glu_alpha, c.glu_beta, c.glu_limit)
        d, _ = M.gemv_fp8(a, c.w_d[e], c.s_d[e], c.b_d[e])
        dense[e] = d
    for (t, s), d in sp.down.items():
        assert np.array_equal(d, dense[int(ids[t, s])][t])
    # a window that holds only half the experts skips the other slots, and
    # its per-slot results are the full chain's results for those slots
    for es in (0, 4):
        half = M.decode_chain(c, es, 4, ids=ids, weights=wts)
        flat = ids.reshape(-1)
        assert np.all((half.slot_row >= 0) == ((flat >= es) & (flat < es + 4)))
        for key, d in half.down.items():
            assert np.array_equal(d, sp.down[key])


def test_glu_special_cases():
    z = F.round_to_bf16(np.zeros(4))
    one = F.round_to_bf16(np.ones(4))
    assert np.all(M.glu(z, one, 1.702, 1.0, 7.0) == 0)
    minus1 = F.round_to_bf16(-np.ones(4))
    assert np.all(F.bf16_to_f32(M.glu(one, minus1, 1.702, 1.0, 7.0)) == 0)     # u + beta == 0
    big = F.round_to_bf16(np.full(4, 50.0))
    assert np.array_equal(M.glu(big, one, 1.702, 1.0, 7.0),
                          M.glu(F.round_to_bf16(np.full(4, 7.0)), one, 1.702, 1.0, 7.0))
    # alpha=1, beta=0, no limit is plain SiLU(g)*u
    g = F.round_to_bf16(np.array([-2.0, -0.5, 0.5, 3.0]))
    u = F.round_to_bf16(np.array([1.5, 2.0, -1.0, 0.25]))
    gv, uv = F.bf16_to_f32(g).astype(np.float64), F.bf16_to_f32(u).astype(np.float64)
    from scipy.special import expit
    assert np.array_equal(M.glu(g, u, 1.0, 0.0, 0.0), F.round_to_bf16(gv * expit(gv) * uv))


def test_gemv_fp8_and_mxfp4_special_cases():
    """One-hot weight rows pick one activation; zero weights leave the bias;
    the per-expert scale and the per-32 scales multiply exactly."""
    rng = np.random.default_rng(16)
    K, N = 64, 5
    act = F.round_to_bf16(rng.standard_normal((2, K)))
    bias = F.round_to_bf16(rng.standard_normal(N))
    w = np.zeros((N, K), np.uint8)
    for n in range(N):
        w[n, 3 * n] = 0x38                           # e4m3 1.0
    y, _ = M.gemv_fp8(act, w, np.float32(2.0), np.zeros(N, np.uint16))
    a = F.bf16_to_f32(act)
    assert np.array_equal(F.bf16_to_f32(y), a[:, 0:3 * N:3] * 2)
    y0, _ = M.gemv_fp8(act, np.zeros((N, K), np.uint8), np.float32(3.0), bias)
    assert np.array_equal(y0, np.broadcast_to(bias, (2, N)))
    wp = np.zeros((N, K // 2), np.uint8)
    for n in range(N):
        wp[n, n] = 0x20                              # e2m1 1.0 in the high nibble: column 2n+1
    sb = np.full((N, K // 32), 128, np.uint8)        # 2^1
    y4, _ = M.gemv_mxfp4(act, wp, sb, np.zeros(N, np.uint16))
    assert np.array_equal(F.bf16_to_f32(y4), a[:, 1:2 * N:2] * 2)


def test_combine_slot_order_in_fp32():
    """The slot order and the fp32 accumulator are fixed by the combine of
    "DeepGEMM FusedMoE on Blackwell (sglang)", section 2.6.1 (a running fp32
    sum over k in order). With weight 1 and rows 2^24, 1, -2^24 in slot order
    the 1 is absorbed (2^24 + 1 rounds to 2^24 in fp32) and the result is 0;
    summed in the reverse order, or in fp64, the result is 1."""
    rows = np.array([[2.0 ** 24], [1.0], [-(2.0 ** 24)]], np.float32)
    w = np.ones((1, 3), np.float32)
    out = M.combine(rows, np.array([[0, 1, 2]]), w)
    assert F.bf16_to_f32(out)[0, 0] == 0.0
    rev = M.combine(rows, np.array([[2, 1, 0]]), w)
    assert F.bf16_to_f32(rev)[0, 0] == 1.0
    # a skipped slot keeps its place: the sum still runs in slot order
    rows4 = np.vstack([rows, [[7.0]]]).astype(np.float32)
    out4 = M.combine(rows4, np.array([[0, -1, 1, 2]]), np.ones((1, 4), np.float32))
    assert F.bf16_to_f32(out4)[0, 0] == 0.0


def _fp32_product_rounded_down_onto(target: float, v: float) -> float:
    """An fp32 w with fl32(w * v) == target while the exact w * v lies above
    target (so the product's rounding drops a positive remainder)."""
    from fractions import Fraction
    w = np.float32(target / v)
    for _ in range(64):
        w = np.nextafter(w, np.float32(-np.inf))
    for _ in range(129):
        if (np.float32(w) * np.float32(v) == np.float32(target)
                and Fraction(float(w)) * Fraction(float(v)) > Fraction(target)):
            return float(w)
        w = np.nextafter(w, np.float32(np.inf))
    raise AssertionError("no such w near target / v")


def test_combine_rounds_product_then_sum():
    """Each slot's product w * v is rounded to fp32 before it is added (two
    roundings, no fused multiply-add). Built so that the difference reaches
    the bf16 output: slot 0 puts 1.0 in the accumulator, slot 1's product
    rounds exactly onto 2^-8 + 2^-24, which makes 1 + 2^-8 + 2^-24 an fp32 tie
    (to even: 1 + 2^-8, itself a bf16 tie that goes to 1.0). Fused, the
    dropped remainder of the product would push the sum above the tie and
    the output to the next bf16 value 1 + 2^-7."""
    from fractions import Fraction
    v = 1.0 + 2.0 ** -7                       # a bf16 value
    target = 2.0 ** -8 + 2.0 ** -24
    w1 = _fp32_product_rounded_down_onto(target, v)
    rows = np.array([[1.0], [v]], np.float32)
    w = np.array([[1.0, w1]], np.float32)
    out = M.combine(rows, np.array([[0, 1]]), w)
    assert F.bf16_to_f32(out)[0, 0] == 1.0
    # fused: 1 + w1 * v exactly lies strictly between the fp32 tie 1 + 2^-8 +
    # 2^-24 and the next fp32 value 1 + 2^-8 + 2^-23, so it rounds up to the
    # latter, which is above the bf16 midpoint 1 + 2^-8
    exact = Fraction(1) + Fraction(w1) * Fraction(v)
    assert Fraction(1) + Fraction(target) < exact < 1 + Fraction(1, 2 ** 8) + Fraction(1, 2 ** 23)
    up = np.array([1.0 + 2.0 ** -8 + 2.0 ** -23], np.float32)
    assert F.bf16_to_f32(F.round_to_bf16(up))[0] == 1.0 + 2.0 ** -7


def test_glu_alpha_is_the_sigmoid_gelu_approximation():
    """With beta = 0, u = 1 and no clamp the decode GLU is g * sigma(alpha g).
    For alpha = 1.702 that is the published sigmoid approximation of GELU
    (Hendrycks and Gimpel, "Gaussian Error Linear Units", section 2:
    x * Phi(x) ~ x * sigma(1.702 x)), whose error stays below 0.021 on the
    whole real line. GELU here is the closed form x * (1 + erf(x / sqrt 2)) / 2.
    sigma(g) in place of sigma(alpha g) misses by about 0.19 at g = 2."""
    import math
    g = F.round_to_bf16(np.linspace(-8.0, 8.0, 2001))
    gv = F.bf16_to_f32(g).astype(np.float64)
    one = F.round_to_bf16(np.ones_like(gv))
    y = F.bf16_to_f32(M.glu(g, one, 1.702, 0.0, 0.0)).astype(np.float64)
    gelu = np.array([x * 0.5 * (1.0 + math.erf(x / math.sqrt(2.0))) for x in gv])
    # approximation error plus one bf16 rounding of the output
    assert np.all(np.abs(y - gelu) <= 0.021 + 2.0 ** -8 * np.abs(gelu))
    plain = F.bf16_to_f32(M.glu(g, one, 1.0, 0.0, 0.0)).astype(np.float64)
    assert np.max(np.abs(plain - gelu)) > 0.15
    # (u + beta), not u * beta or u alone: with u = 0 the factor is beta
    zero = F.round_to_bf16(np.zeros_like(gv))
    y_b = F.bf16_to_f32(M.glu(g, zero, 1.702, 1.0, 0.0)).astype(np.float64)
    assert np.array_equal(y_b, y)
