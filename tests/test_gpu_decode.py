"""GPU parity of the sparse decode path (route -> sparse GEMV gate_up with
fused bias and GLU -> sparse GEMV down with bias -> skip-combine) against
the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import moe as M
from tests.gpu_helpers import BF16_SENT, dev, dev_bf16, end_to_end_ok, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import mixture_experts_ffn_scatter_amd as pkg
    pkg.lib()
    return pkg.ops


def _dev_case(c, sl):
    if c.wfmt == "fp8":
        return (dev(c.w_gu[sl]), dev(c.s_gu[sl]), dev_bf16(c.b_gu[sl]),
                dev(c.w_d[sl]), dev(c.s_d[sl]), dev_bf16(c.b_d[sl]))
    return (dev(c.w_gu[sl]), dev(c.s_gu[sl]), dev_bf16(c.b_gu[sl]),
            dev(c.w_d[sl]), dev(c.s_d[sl]), dev_bf16(c.b_d[sl]))


def _bf(bits):
    return F.bf16_to_f32(bits).astype(np.float64)


def _check_stage(got, want, rel=2.0 ** -6):
    """A GEMV output may differ from the oracle by its fp32 accumulation
    order, which can move the bf16 rounding by one step."""
    g, w = _bf(got), _bf(want)
    assert np.all(np.abs(g - w) <= rel * np.abs(w) + 1e-2 * np.abs(w).mean() + 1e-30)


@pytest.mark.parametrize("wfmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_decode_small_shapes(ops, wfmt, T):
    """H=256 keeps the oracle instant; 8 experts of 32 hold weights and
    routes to the others are skipped (a local window)."""
    say(f"decode small {wfmt} T={T}")
    c = W.decode(T=T, H=256, experts=8, wfmt=wfmt)
    ids, wts = M.route_softmax(c.logits, c.k)
    ref = M.decode_chain(c, 0, 8, ids=ids, weights=wts)
    buf = ops.alloc_decode(T, c.k, c.H, fill=True)
    y = ops.moe_ffn_decode(dev_bf16(c.x), dev(ids), dev(wts), 0, 8, wfmt, *_dev_case(c, slice(0, 8)),
                           buf)
    slot_row = host(buf.slot_row)
    assert np.array_equal(slot_row, ref.slot_row)
    act, down = host(buf.act), host(buf.down)
    for (t, s), a in ref.act.items():
        _check_stage(act[t * c.k + s], a)
    nonlocal_rows = np.flatnonzero(ref.slot_row < 0)
    assert np.all(act[nonlocal_rows] == BF16_SENT) and np.all(down[nonlocal_rows] == BF16_SENT)
    # down stage from the GPU's own activations, then the combine bit-exactly
    for (t, s) in ref.down:
        e = int(ids[t, s])
        q = t * c.k + s
        if wfmt == "fp8":
            d, _ = M.gemv_fp8(act[q:q + 1], c.w_d[e], c.s_d[e], c.b_d[e])
        else:
            d, _ = M.gemv_mxfp4(act[q:q + 1], c.w_d[e], c.s_d[e], c.b_d[e])
        _check_stage(down[q], d[0])
    rows = F.bf16_to_f32(down)
    assert np.array_equal(host(y), M.combine(rows, slot_row, wts, 1.0))
    ok, mx, mean = end_to_end_ok(host(y), ref.out)
    assert ok, (mx, mean)


def test_decode_windows_skip_not_zero(ops):
    """Two 16-expert windows (a tensor-parallel split of 32 experts): each
    window skips the other's slots; the two partial sums add up."""
    say("decode windows 0..15 / 16..31")
    c = W.decode(T=4, H=256, experts=32)
    ids, wts = M.route_softmax(c.logits, c.k)
    parts = []
    for es in (0, 16):
        buf = ops.alloc_decode(4, c.k, c.H, fill=True)
        ops.moe_ffn_decode(dev_bf16(c.x), dev(ids), dev(wts), es, 16, "fp8",
                           *_dev_case(c, slice(es, es + 16)), buf)
        parts.append(_bf(host(buf.out)))
        ref = M.decode_chain(c, es, 16, ids=ids, weights=wts)
        ok, mx, mean = end_to_end_ok(host(buf.out), ref.out)
        assert ok, (es, mx, mean)
    full = M.decode_chain(c, 0, 32, ids=ids, weights=wts)
    total = parts[0] + parts[1]
    assert np.allclose(total, _bf(full.out), rtol=2e-2, atol=1e-2 * np.abs(_bf(full.out)).max())


@pytest.mark.parametrize("wfmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("H", [2880, 4608])
def test_decode_wide_rows_many_slots(ops, wfmt, H):
    """Full-width rows (K = 2880: the 180 weight chunks of a row end inside
    the block's third wave; K = 4608: two chunks per thread) and every
    token routed to both local experts, so each expert serves 8 slots in
    several slot batches."""
    say(f"decode wide {wfmt} H={H}")
    c = W.decode(T=8, H=H, experts=2, wfmt=wfmt)
    c.logits = c.logits.copy()
    c.logits[:, :2] += 8.0
    ids, wts = M.route_softmax(c.logits, c.k)
    assert np.all((ids == 0).any(axis=1) & (ids == 1).any(axis=1))
    ref = M.decode_chain(c, 0, 2, ids=ids, weights=wts)
    buf = ops.alloc_decode(8, c.k, c.H, fill=True)
    y = ops.moe_ffn_decode(dev_bf16(c.x), dev(ids), dev(wts), 0, 2, wfmt, *_dev_case(c, slice(0, 2)),
                           buf)
    slot_row = host(buf.slot_row)
    assert np.array_equal(slot_row, ref.slot_row)
    act = host(buf.act)
    for (t, s), a in ref.act.items():
        _check_stage(act[t * c.k + s], a)
    ok, mx, mean = end_to_end_ok(host(y), ref.out)
    assert ok, (mx, mean)
