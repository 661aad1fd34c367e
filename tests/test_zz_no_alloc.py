"""moe_scatter_endpoints_noalloc (the static-scratch form of the scatter, for
callers that cannot allocate) against moe_scatter_endpoints with a caller
workspace: byte-identical expert_ends, route_row, xq and xs (padding
sentinels untouched) on two calls in a row, the second with smaller sizes,
so the second call runs over the scratch contents the first one left."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe as M
from tests.gpu_helpers import dev, dev_bf16, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import mixture_experts_ffn_scatter_amd as pkg
    pkg.lib()
    return pkg.ops


def _both(ops, ids, x_bits, expert_start, E_local, A, M_cap):
    T, k = ids.shape
    H = x_bits.shape[1]
    outs = []
    for noalloc in (False, True):
        buf = ops.alloc_grouped(T, k, E_local, M_cap, H, 128, fill=True)
        buf.expert_ends.fill_(-7)
        buf.route_row.fill_(-7)
        if noalloc:
            ops.moe_scatter_endpoints_noalloc(dev(ids), expert_start, E_local, A, dev_bf16(x_bits),
                                              buf.expert_ends, buf.route_row, buf.xq, buf.xs)
        else:
            ops.moe_scatter_endpoints(dev(ids), expert_start, E_local, A, dev_bf16(x_bits),
                                      buf.expert_ends, buf.route_row, buf.xq, buf.xs, buf.workspace)
        outs.append([host(buf.expert_ends), host(buf.route_row), host(buf.xq), host(buf.xs)])
    return outs


def test_noalloc_scatter_equals_workspace_scatter_twice(ops):
    # first call: the prefill EP group (4,096 tokens x top-6, 32 local experts,
    # H = 4,096); it fills 65 x 32 counters of the scratch
    c = W.prefill(with_weights=False)
    ids, _ = M.route_softmax(c.logits, c.k)
    say("no-alloc scatter: EP group 4096 x 6 -> 32 experts")
    a, b = _both(ops, ids, c.x, 0, c.E_local, c.A, c.M_cap)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    # second call, smaller: 64 tokens x top-2 over a window of 6 of 8 experts
    # with -1 ids, A = 16; its 2 x 6 counters overlap what the first call left
    t = W.tiny(seed=5)
    ids2, _ = M.route_softmax(t.logits, t.k)
    ids2 = ids2.copy()
    ids2[7, 0] = -1
    M_cap2 = W.capacity(t.T, t.k, 6, 16)
    say("no-alloc scatter: second call, 64 x 2 -> window 1..6, A=16")
    a, b = _both(ops, ids2, t.x, 1, 6, 16, M_cap2)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    sc = M.scatter_routes(ids2, 1, 6, 16)
    assert np.array_equal(b[0], sc.end.astype(np.int32)) and np.array_equal(b[1], sc.route_row)
