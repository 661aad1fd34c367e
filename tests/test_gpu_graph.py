"""HIP-graph capture of the prefill chain ("Blackwell FP4 MoE: live-row
boundary", section 3: the metadata lives on the device, so a captured FFN can
be replayed while the routing and every expert count change underneath it).

One graph of route -> scatter -> GEMM1 -> act-quant -> GEMM2 -> combine is
captured on fixed buffers, then replayed with new logits written in place
(including a routing whose expert loads are the reverse of the captured
one). Eager runs of the same chain on separate buffers happen between the
replays; every replay must equal its eager run bit for bit, and the first
one must match the oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe as M
from tests.gpu_helpers import dev, dev_bf16, end_to_end_ok, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import mixture_experts_ffn_scatter_amd as pkg
    pkg.lib()
    return pkg.ops


def _logit_sets(c, n):
    rng = np.random.default_rng(4242)
    sets = [c.logits]
    for _ in range(n - 2):
        sets.append(rng.standard_normal(c.logits.shape, dtype=np.float32))
    # reversed loads: the experts' columns in reverse order move the hot
    # experts of the captured routing to the cold end and vice versa
    sets.append(np.ascontiguousarray(c.logits[:, ::-1]))
    return sets


@pytest.mark.parametrize("fused", [False, True])
def test_prefill_chain_graph_replays_follow_new_routing(ops, fused):
    c = W.tiny()
    w = c.weights
    pack13 = ops.moe_pack_mx_weights_gateup if fused else ops.moe_pack_mx_weights
    prefill = ops.moe_ffn_prefill_fused if fused else ops.moe_ffn_prefill
    w13p, s13p = pack13(dev(w.w13), dev(w.s13))
    w2p, s2p = ops.moe_pack_mx_weights(dev(w.w2), dev(w.s2))
    x = dev_bf16(c.x)

    def buffers():
        logits = torch.empty((c.T, c.E), dtype=torch.float32, device="cuda")
        ids = torch.empty((c.T, c.k), dtype=torch.int32, device="cuda")
        wts = torch.empty((c.T, c.k), dtype=torch.float32, device="cuda")
        return logits, ids, wts, ops.alloc_grouped(c.T, c.k, c.E, c.M_cap, c.H, c.I, fill=True)

    def chain(logits, ids, wts, buf):
        ops.moe_route(logits, c.k, "softmax", None, ids, wts)
        prefill(x, ids, wts, 0, c.A, w13p, s13p, w2p, s2p, buf)

    g_logits, g_ids, g_wts, g_buf = buffers()
    e_logits, e_ids, e_wts, e_buf = buffers()
    g_logits.copy_(dev(c.logits))
    say(f"capture the prefill chain (fused={fused})")
    graph = ops.capture_graph(lambda: chain(g_logits, g_ids, g_wts, g_buf))
    torch.cuda.synchronize()
    for r, lg in enumerate(_logit_sets(c, 4)):
        say(f"graph replay {r}")
        g_logits.copy_(dev(lg))
        graph.replay()
        torch.cuda.synchronize()
        y_graph = host(g_buf.out).copy()
        ends_graph = host(g_buf.expert_ends).copy()
        # eager work between the replays, on separate buffers
        e_logits.copy_(dev(lg))
        chain(e_logits, e_ids, e_wts, e_buf)
        torch.cuda.synchronize()
        assert np.array_equal(ends_graph, host(e_buf.expert_ends))
        assert np.array_equal(host(g_ids), host(e_ids))
        assert np.array_equal(y_graph, host(e_buf.out)), f"replay {r} differs from eager"
        ids, wts = M.route_softmax(lg, c.k)
        assert np.array_equal(host(g_ids), ids)
        if r in (0, 3):
            ref = M.prefill_expert_major(c.x, ids, wts, 0, c.E, c.A, c.I, w.w13, w.s13, w.w2, w.s2)
            ok, mx, mean = end_to_end_ok(y_graph, ref.out)
            assert ok, (r, mx, mean)
    # the reversed routing really moved the loads
    counts0 = np.bincount(M.route_softmax(c.logits, c.k)[0].ravel(), minlength=c.E)
    counts3 = np.bincount(M.route_softmax(np.ascontiguousarray(c.logits[:, ::-1]), c.k)[0].ravel(),
                          minlength=c.E)
    assert np.array_equal(counts0[::-1], counts3)
