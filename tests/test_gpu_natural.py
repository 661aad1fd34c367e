"""GPU: the grouped GEMMs on checkpoint-layout weights (no packing) against
the packed forms, through the C ABI. Both read the same weight bytes and sum
the same products in the same order, so their outputs must be equal bit for
bit; the packed forms are pinned to the oracle by the prefill tests. One
case also checks the natural form against the oracle directly."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import moe as M
from tests.gpu_helpers import (BF16_SENT, BYTE_SENT, WORD_SENT, dev, dev_bf16, gemm_within_bound,
                               host, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import mixture_experts_ffn_scatter_amd as pkg
    pkg.lib()
    return pkg.ops


def _layout(counts, A):
    ends, prev = [], 0
    for cnt in counts:
        start = ((prev + A - 1) // A) * A
        ends.append(start + cnt)
        prev = start + cnt
    return ends, max(((prev + A - 1) // A) * A, A)


def _acts(rng, M_cap, K):
    xq = rng.integers(0, 256, size=(M_cap, K), dtype=np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x3C                      # no E4M3 NaN codes
    xsb = rng.integers(118, 131, size=(M_cap, K // 32), dtype=np.uint8)
    return xq, xsb, np.ascontiguousarray(F.pack_ue8m0_words(xsb).T)


@pytest.mark.parametrize("K,N,seed", [(128, 128, 1), (256, 384, 2), (384, 640, 3), (1152, 256, 4)])
def test_natural_gemm_equals_packed(ops, K, N, seed):
    """Experts with no rows, one full chunk, a chunk plus one row, single
    rows, several chunks; 1-9 k-steps; partial 256-column tiles."""
    say(f"natural vs packed GEMM K={K} N={N}")
    rng = np.random.default_rng(seed)
    counts = [0, 128, 129, 1, 300, 0, 17]
    ends, M_cap = _layout(counts, 128)
    xq, xsb, xs = _acts(rng, M_cap, K)
    w = rng.integers(0, 256, size=(len(counts), N, K // 2), dtype=np.uint8)
    ws = rng.integers(118, 131, size=(len(counts), N, K // 32), dtype=np.uint8)
    wp, sp = ops.moe_pack_mx_weights(dev(w), dev(ws))
    ends_d = dev(np.asarray(ends, np.int32))
    outs = []
    for natural in (False, True):
        out = torch.full((M_cap, N), BF16_SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        if natural:
            ops.moe_grouped_gemm2_natural(dev(xq), dev(xs), ends_d, 128, dev(w), dev(ws), out)
        else:
            ops.moe_grouped_gemm2(dev(xq), dev(xs), ends_d, 128, wp, sp, out)
        outs.append(host(out))
    assert np.array_equal(outs[0], outs[1])
    # and the natural form against the oracle on one expert of several chunks
    start = ((ends[3] + 127) // 128) * 128
    rows = np.arange(start, ends[4])
    _, exact, tsum = M.mx_gemm(xq[rows], xsb[rows], w[4], ws[4])
    bm = M.block_max_bound(xq[rows], xsb[rows], w[4], ws[4])
    ok, _, _ = gemm_within_bound(outs[1][rows], exact, tsum, K, bm)
    assert ok.all()


@pytest.mark.parametrize("I,clamp", [(128, 0.0), (256, 6.0), (384, 0.0)])
def test_natural_fused_gemm1_equals_packed(ops, I, clamp):
    """The fused GEMM1 + act-quant: the gate/up interleave of the packed form
    becomes an address mapping; hq and hs byte-equal to the packed fused
    form, and the plain GEMM1 on natural weights equal to the packed one."""
    say(f"natural vs packed fused GEMM1 I={I}")
    rng = np.random.default_rng(I)
    H = 256
    counts = [0, 128, 129, 1, 300, 0, 17]
    ends, M_cap = _layout(counts, 128)
    xq, _, xs = _acts(rng, M_cap, H)
    w13 = rng.integers(0, 256, size=(len(counts), 2 * I, H // 2), dtype=np.uint8)
    s13 = rng.integers(118, 128, size=(len(counts), 2 * I, H // 32), dtype=np.uint8)
    gp, gs = ops.moe_pack_mx_weights_gateup(dev(w13), dev(s13))
    wp, sp = ops.moe_pack_mx_weights(dev(w13), dev(s13))
    ends_d = dev(np.asarray(ends, np.int32))
    res = []
    for natural in (False, True):
        hq = torch.full((M_cap, I), BYTE_SENT, dtype=torch.uint8, device="cuda")
        hs = torch.full((I // 128, M_cap), int(WORD_SENT), dtype=torch.int32, device="cuda")
        gu = torch.full((M_cap, 2 * I), BF16_SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        if natural:
            ops.moe_grouped_gemm1_act_quant_natural(dev(xq), dev(xs), ends_d, 128, dev(w13),
                                                    dev(s13), clamp, hq, hs)
            ops.moe_grouped_gemm1_natural(dev(xq), dev(xs), ends_d, 128, dev(w13), dev(s13), gu)
        else:
            ops.moe_grouped_gemm1_act_quant(dev(xq), dev(xs), ends_d, 128, gp, gs, clamp, hq, hs)
            ops.moe_grouped_gemm1(dev(xq), dev(xs), ends_d, 128, wp, sp, gu)
        res.append((host(hq), host(hs), host(gu)))
    for a, b in zip(*res):
        assert np.array_equal(a, b)


def test_natural_gemms_equal_packed_ep_share(ops):
    """The EP-share layer's GEMM1 + act-quant and GEMM2 on natural weights,
    every buffer byte-equal to the packed forms (live rows and padding)."""
    c = W.prefill()
    w = c.weights
    ids, wts = M.route_softmax(c.logits, c.k)
    buf = ops.alloc_grouped(c.T, c.k, c.E_local, c.M_cap, c.H, c.I, fill=True)
    ops.moe_scatter_endpoints(dev(ids), 0, c.E_local, c.A,
                              torch.from_numpy(c.x.view(np.int16)).cuda().view(torch.bfloat16),
                              buf.expert_ends, buf.route_row, buf.xq, buf.xs, buf.workspace)
    gp, gs = ops.moe_pack_mx_weights_gateup(dev(w.w13), dev(w.s13))
    w2p, s2p = ops.moe_pack_mx_weights(dev(w.w2), dev(w.s2))
    res = []
    for natural in (False, True):
        say(f"EP share, natural={natural}")
        hq = torch.full_like(buf.hq, BYTE_SENT)
        hs = torch.full_like(buf.hs, int(WORD_SENT))
        down = torch.full((c.M_cap, c.H), BF16_SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        if natural:
            ops.moe_grouped_gemm1_act_quant_natural(buf.xq, buf.xs, buf.expert_ends, c.A,
                                                    dev(w.w13), dev(w.s13), 0.0, hq, hs)
            ops.moe_grouped_gemm2_natural(hq, hs, buf.expert_ends, c.A, dev(w.w2), dev(w.s2), down)
        else:
            ops.moe_grouped_gemm1_act_quant(buf.xq, buf.xs, buf.expert_ends, c.A, gp, gs, 0.0,
                                            hq, hs)
            ops.moe_grouped_gemm2(hq, hs, buf.expert_ends, c.A, w2p, s2p, down)
        res.append((host(hq), host(hs), host(down)))
        torch.cuda.empty_cache()
    for a, b in zip(*res):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("case,clamp,scale", [("tiny", 7.0, 2.5), ("prefill", 0.0, 1.0)])
def test_natural_chain_equals_fused_chain(ops, case, clamp, scale):
    """moe_ffn_prefill_natural (checkpoint-layout weights, no packing) equals
    moe_ffn_prefill_fused on the packed weights in every buffer, byte for byte."""
    c = W.tiny() if case == "tiny" else W.prefill()
    w = c.weights
    ids, wts = M.route_softmax(c.logits, c.k)
    say(f"natural chain vs fused chain: {case}")
    outs = []
    for natural in (False, True):
        buf = ops.alloc_grouped(c.T, c.k, c.E_local, c.M_cap, c.H, c.I, fill=True)
        if natural:
            ops.moe_ffn_prefill_natural(dev_bf16(c.x), dev(ids), dev(wts), c.expert_start, c.A,
                                        dev(w.w13), dev(w.s13), dev(w.w2), dev(w.s2), buf,
                                        clamp_limit=clamp, routed_scale=scale)
        else:
            g = ops.moe_pack_mx_weights_gateup(dev(w.w13), dev(w.s13))
            d = ops.moe_pack_mx_weights(dev(w.w2), dev(w.s2))
            ops.moe_ffn_prefill_fused(dev_bf16(c.x), dev(ids), dev(wts), c.expert_start, c.A,
                                      *g, *d, buf, clamp_limit=clamp, routed_scale=scale)
        outs.append((host(buf.hq), host(buf.hs), host(buf.down), host(buf.out)))
        del buf
        torch.cuda.empty_cache()
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
