"""GPU parity of the masked (E, m_pad, K) slab layout against the CPU oracle,
through the C ABI: the masked scatter (masked_m, route rows, FP8 codes and
per-expert MN-major scale words, bit-exact), both masked GEMMs within the
accumulation bound, the varlen act-quant bit-exact on the GPU's own gate/up
rows, the fused GEMM1 + act-quant byte-equal to the two calls, the combine
over the slab's rows bit-exact, and the chain end to end. Every slab is
seeded with sentinels that must survive outside the live rows."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import moe as M
from tests.gpu_helpers import (BF16_SENT, BYTE_SENT, WORD_SENT, dev, dev_bf16, end_to_end_ok,
                               gemm_within_bound, host, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import mixture_experts_ffn_scatter_amd as pkg
    pkg.lib()
    return pkg.ops


def _slab_live(masked_m, m_pad):
    E = masked_m.shape[0]
    live = np.zeros(E * m_pad, bool)
    for e in range(E):
        live[e * m_pad:e * m_pad + int(masked_m[e])] = True
    return live


def _check_chain(ops, x, ids, wts, es, E_local, m_pad, I, w13, s13, w2, s2, clamp=0.0,
                 scale=1.0, workers=1):
    """Stage by stage, each stage fed the GPU's own input to it."""
    T, k = ids.shape
    H = x.shape[1]
    ref = M.prefill_masked(x, ids, wts, es, E_local, m_pad, I, w13, s13, w2, s2, clamp=clamp,
                           routed_scale=scale, workers=workers)
    sc = ref.scatter
    rows = sc.route_row[sc.local_routes].astype(np.int64)      # slab row of each placed route
    live = _slab_live(sc.masked_m, m_pad)
    buf = ops.alloc_masked(T, k, E_local, m_pad, H, I, fill=True)
    say(f"masked scatter T={T} k={k} E_local={E_local} m_pad={m_pad} H={H}")
    ops.moe_scatter_masked(dev(ids), es, dev_bf16(x), buf.masked_m, buf.route_row, buf.xq, buf.xs,
                           buf.workspace)
    assert np.array_equal(host(buf.masked_m), sc.masked_m)
    assert np.array_equal(host(buf.route_row), sc.route_row)
    xq = host(buf.xq).reshape(E_local * m_pad, H)
    assert np.array_equal(xq[rows], ref.xq)
    assert np.all(xq[~live] == BYTE_SENT)
    want_xs = M.scales_slab(ref.xb, rows, E_local, m_pad, fill=WORD_SENT)
    assert np.array_equal(host(buf.xs), want_xs)

    w13p, s13p = ops.moe_pack_mx_weights(dev(w13), dev(s13))
    w2p, s2p = ops.moe_pack_mx_weights(dev(w2), dev(s2))
    say("masked gemm1")
    ops.moe_grouped_gemm1_masked(buf.xq, buf.xs, buf.masked_m, w13p, s13p, buf.gateup)
    gu = host(buf.gateup).reshape(E_local * m_pad, 2 * I)
    for e in np.unique(sc.local_expert):
        sel = np.flatnonzero(sc.local_expert == e)
        bm = M.block_max_bound(ref.xq[sel], ref.xb[sel], w13[e], s13[e])
        ok, _, _ = gemm_within_bound(gu[rows[sel]], ref.gateup_exact[sel], ref.gateup_tsum[sel],
                                     H, bm)
        assert ok.all(), f"gemm1 expert {e}: {np.count_nonzero(~ok)} of {ok.size} outside bound"
    assert np.all(gu[~live] == BF16_SENT)

    say("masked act-quant on the GPU's gate/up")
    ops.moe_act_quant_masked(buf.gateup, buf.masked_m, clamp, buf.hq, buf.hs)
    hq = host(buf.hq).reshape(E_local * m_pad, I)
    q, b = M.act_quant_rows(gu[rows], I, clamp)
    assert np.array_equal(hq[rows], q)
    assert np.all(hq[~live] == BYTE_SENT)
    hs = host(buf.hs)
    assert np.array_equal(hs, M.scales_slab(b, rows, E_local, m_pad, fill=WORD_SENT))

    say("masked fused gemm1 + act-quant")
    g13p, g13s = ops.moe_pack_mx_weights_gateup(dev(w13), dev(s13))
    hq2 = torch.full_like(buf.hq, BYTE_SENT)
    hs2 = torch.full_like(buf.hs, int(WORD_SENT))
    ops.moe_grouped_gemm1_act_quant_masked(buf.xq, buf.xs, buf.masked_m, g13p, g13s, clamp, hq2, hs2)
    assert np.array_equal(host(hq2).reshape(E_local * m_pad, I), hq)
    assert np.array_equal(host(hs2), hs)

    say("masked gemm2")
    ops.moe_grouped_gemm2_masked(buf.hq, buf.hs, buf.masked_m, w2p, s2p, buf.down)
    dn = host(buf.down).reshape(E_local * m_pad, H)
    for e in np.unique(sc.local_expert):
        sel = np.flatnonzero(sc.local_expert == e)
        _, exact, tsum = M.mx_gemm(q[sel], b[sel], w2[e], s2[e])
        bm = M.block_max_bound(q[sel], b[sel], w2[e], s2[e])
        ok, _, _ = gemm_within_bound(dn[rows[sel]], exact, tsum, I, bm)
        assert ok.all(), f"gemm2 expert {e}: {np.count_nonzero(~ok)} of {ok.size} outside bound"
    assert np.all(dn[~live] == BF16_SENT)

    say("combine over the slab rows")
    ops.moe_combine(buf.down.view(E_local * m_pad, H), buf.route_row, dev(wts), scale, buf.out)
    out = host(buf.out)
    assert np.array_equal(out, M.combine(F.bf16_to_f32(dn), sc.route_row, wts, scale))
    ok, mx, mean = end_to_end_ok(out, ref.out)
    assert ok, (mx, mean)
    return ref, out


def test_masked_chain_tiny(ops):
    c = W.tiny()
    ids, wts = M.route_softmax(c.logits, c.k)
    counts = np.bincount(ids.reshape(-1), minlength=c.E)
    m_pad = (int(counts.max()) + 3) // 4 * 4 + 4
    w = c.weights
    _check_chain(ops, c.x, ids, wts, 0, c.E, m_pad, c.I, w.w13, w.s13, w.w2, w.s2)


def test_masked_chain_overflowing_slabs(ops):
    """m_pad below the busiest experts' counts: the routes past a full slab
    are not placed (row -1) and leave the output."""
    c = W.tiny()
    ids, wts = M.route_softmax(c.logits, c.k)
    w = c.weights
    ref, _ = _check_chain(ops, c.x, ids, wts, 0, c.E, 8, c.I, w.w13, w.s13, w.w2, w.s2)
    assert int(ref.scatter.counts.max()) > 8
    assert np.count_nonzero(ref.scatter.route_row == -1) > 0


def test_masked_chain_window_clamp_scale(ops):
    """Local window of 4 of 8 experts, a -1 slot, clamp 6, routed scale 0.5."""
    c = W.tiny(seed=77, T=40)
    ids, wts = M.route_softmax(c.logits, c.k)
    ids = ids.copy()
    ids[3, 1] = -1
    w = c.weights
    sl = slice(2, 6)
    ref, out = _check_chain(ops, c.x, ids, wts, 2, 4, 40, c.I, w.w13[sl], w.s13[sl], w.w2[sl],
                            w.s2[sl], clamp=6.0, scale=0.5)
    no_local = ~np.any((ids >= 2) & (ids < 6), axis=1)
    assert np.all(out[no_local] == 0)


def test_masked_chain_multi_chunk_ragged(ops):
    """Experts with 0, 2 and 440-666 rows (several 128-row chunks and a
    ragged last one), m_pad not a multiple of 128, H = 512,
    I = 256 (two n-tiles of GEMM1, one of the act-quant's 512-column chunks)."""
    rng = np.random.default_rng(2024)
    T, k, E, H, I = 700, 3, 6, 512, 256
    p = np.array([0.0, 0.5, 0.2, 0.15, 0.149, 0.001])
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    wts = rng.random((T, k), dtype=np.float32)
    x = W.normal_bf16(rng, (T, H))
    w = W._mx_weights(rng, E, H, I)
    _check_chain(ops, x, ids, wts, 0, E, 700, I, w.w13, w.s13, w.w2, w.s2)


def test_masked_scatter_long_token_blocks(ops):
    """5,000 tokens: more token blocks than the rows kernel scans itself, so
    the one-block count-and-scan launch runs first; slabs overflow too."""
    rng = np.random.default_rng(5)
    T, k, E, H = 5000, 2, 8, 128
    ids = np.stack([rng.choice(E + 2, size=k, replace=False) for _ in range(T)]).astype(np.int32) - 1
    x = W.normal_bf16(rng, (T, H))
    for m_pad in (1300, 1000):
        say(f"masked scatter T={T} m_pad={m_pad}")
        sc = M.scatter_masked(ids, 0, E, m_pad)
        buf = ops.alloc_masked(T, k, E, m_pad, H, 128, fill=True)
        ops.moe_scatter_masked(dev(ids), 0, dev_bf16(x), buf.masked_m, buf.route_row, buf.xq,
                               buf.xs, buf.workspace)
        assert np.array_equal(host(buf.masked_m), sc.masked_m)
        assert np.array_equal(host(buf.route_row), sc.route_row)
        rows = sc.route_row[sc.local_routes].astype(np.int64)
        q, b = M.quant_rows(x[sc.local_routes // k])
        xq = host(buf.xq).reshape(E * m_pad, H)
        assert np.array_equal(xq[rows], q)
        assert np.all(xq[~_slab_live(sc.masked_m, m_pad)] == BYTE_SENT)
        assert np.array_equal(host(buf.xs), M.scales_slab(b, rows, E, m_pad, fill=WORD_SENT))
    assert int(sc.counts.max()) > 1000


def test_masked_degenerate_calls(ops):
    """No tokens: masked_m all zero. No local route: nothing placed, the
    GEMMs and the act-quant write nothing, the output is zero."""
    H, I, E, m_pad, k = 256, 128, 4, 16, 2
    buf = ops.alloc_masked(0, k, E, m_pad, H, I, fill=True)
    buf.masked_m.fill_(-7)
    ops.moe_scatter_masked(torch.empty((0, k), dtype=torch.int32, device="cuda"), 0,
                           torch.empty((0, H), dtype=torch.bfloat16, device="cuda"), buf.masked_m,
                           buf.route_row, buf.xq, buf.xs, buf.workspace)
    assert np.all(host(buf.masked_m) == 0)

    rng = np.random.default_rng(9)
    T = 24
    ids = rng.integers(10, 20, size=(T, k)).astype(np.int32)
    x = W.normal_bf16(rng, (T, H))
    w = W._mx_weights(rng, E, H, I)
    buf = ops.alloc_masked(T, k, E, m_pad, H, I, fill=True)
    y = ops.moe_ffn_prefill_masked(dev_bf16(x), dev(ids), dev(rng.random((T, k), dtype=np.float32)),
                                   0, *ops.moe_pack_mx_weights(dev(w.w13), dev(w.s13)),
                                   *ops.moe_pack_mx_weights(dev(w.w2), dev(w.s2)), buf)
    assert np.all(host(buf.masked_m) == 0) and np.all(host(buf.route_row) == -1)
    assert np.all(host(buf.gateup) == BF16_SENT) and np.all(host(buf.hq) == BYTE_SENT)
    assert np.all(host(buf.down) == BF16_SENT)
    assert np.all(host(y) == 0)


def test_masked_ep_share_layer_end_to_end(ops):
    """The prefill EP share (4,096-token group, 32 local experts, H = 4,096,
    I = 2,048) on slabs of m_pad = 4,096 rows (the group's token count, the
    pages' default capacity): masked_m and route rows bit-exact, the fused
    chain end to end against the oracle, and bitwise equal on a rerun."""
    c = W.prefill()
    w = c.weights
    ids, wts = M.route_softmax(c.logits, c.k)
    m_pad = c.T
    say("masked EP share: oracle")
    ref = M.prefill_masked(c.x, ids, wts, 0, c.E_local, m_pad, c.I, w.w13, w.s13, w.w2, w.s2,
                           workers=16)
    g13p, g13s = ops.moe_pack_mx_weights_gateup(dev(w.w13), dev(w.s13))
    w2p, s2p = ops.moe_pack_mx_weights(dev(w.w2), dev(w.s2))
    outs = []
    for rep in range(2):
        say(f"masked EP share: fused chain, run {rep}")
        buf = ops.alloc_masked(c.T, c.k, c.E_local, m_pad, c.H, c.I)
        y = ops.moe_ffn_prefill_masked(dev_bf16(c.x), dev(ids), dev(wts), 0, g13p, g13s, w2p, s2p,
                                       buf, fused=True)
        outs.append(host(y))
        if rep == 0:
            assert np.array_equal(host(buf.masked_m), ref.scatter.masked_m)
            assert np.array_equal(host(buf.route_row), ref.scatter.route_row)
        del buf
        torch.cuda.empty_cache()
    assert np.array_equal(outs[0].view(np.int16), outs[1].view(np.int16))
    ok, mx, mean = end_to_end_ok(outs[0], ref.out)
    say(f"masked EP share e2e max {mx:.3e} mean {mean:.3e}")
    assert ok, (mx, mean)
