"""GPU parity of the group-128 activation recipe (one UE8M0 byte per 128
columns, four groups per packed word) through the C ABI: the scatter and the
live-row act-quant bit-exact against the oracle, padding untouched; both
grouped GEMMs within the GEMM bound of the oracle with the group's scale on
each of its 32-column blocks."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import moe as M
from tests.gpu_helpers import (BF16_SENT, BYTE_SENT, WORD_SENT, actquant_case, dev, dev_bf16, gemm_within_bound,
                               host, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import mixture_experts_ffn_scatter_amd as pkg
    pkg.lib()
    return pkg.ops


def _words(K):
    return (K + 511) // 512


@pytest.mark.parametrize("T,k,E,E_local,H,A", [(300, 4, 16, 16, 640, 128), (513, 6, 64, 24, 2048, 32)])
def test_scatter_g128(ops, T, k, E, E_local, H, A):
    """H = 640: the second word holds one group and three zero bytes."""
    say(f"scatter g128 T={T} k={k} E_local={E_local} H={H}")
    rng = np.random.default_rng(T + H)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = F.round_to_bf16(rng.standard_normal((T, H)) * np.exp2(rng.uniform(-6, 6, size=(T, 1))))
    M_cap = M.align_up(T * k + E_local * A, 128)
    ends = torch.full((E_local,), -7, dtype=torch.int32, device="cuda")
    rr = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    xq = torch.full((M_cap, H), BYTE_SENT, dtype=torch.uint8, device="cuda")
    xs = torch.full((_words(H), M_cap), int(WORD_SENT), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(ops.moe_scatter_workspace_bytes(T, k, E_local), 1), dtype=torch.uint8,
                     device="cuda")
    ops.moe_scatter_endpoints(dev(ids), 0, E_local, A, dev_bf16(x), ends, rr, xq, xs, ws, group=128)
    ends, rr, xq, xs = host(ends), host(rr), host(xq), host(xs)
    sc = M.scatter_routes(ids, 0, E_local, A)
    assert np.array_equal(ends, sc.end.astype(np.int32))
    assert np.array_equal(rr, sc.route_row)
    rows = sc.route_row[sc.local_routes]
    q, b = M.quant_rows_g128(x[sc.local_routes // k])
    assert np.array_equal(xq[rows], q)
    assert np.array_equal(xs[:, rows].T, M.pack_g128_words(b))
    live = M.live_row_mask(sc.start, sc.end, M_cap)
    assert np.all(xq[~live] == BYTE_SENT) and np.all(xs[:, ~live] == WORD_SENT)


@pytest.mark.parametrize("I,clamp,small", [(640, 0.0, True), (384, 6.0, True), (2048, 0.0, False)])
def test_act_quant_liverows_g128(ops, I, clamp, small):
    say(f"act-quant g128 I={I} clamp={clamp}")
    if small:
        counts = np.array([5, 0, 17, 1, 0, 9, 40], np.int64)
        case = actquant_case(counts=counts, E_local=7, I=I, A=8, M_cap=128)
    else:
        case = actquant_case()
    start, end = M.endpoints(case.counts, case.A)
    hq = torch.full((case.M_cap, case.I), BYTE_SENT, dtype=torch.uint8, device="cuda")
    hs = torch.full((_words(case.I), case.M_cap), int(WORD_SENT), dtype=torch.int32, device="cuda")
    ops.moe_act_quant_liverows(dev_bf16(case.gateup), dev(end.astype(np.int32)), case.A, clamp, hq,
                               hs, group=128)
    hq, hs = host(hq), host(hs)
    live = M.live_row_mask(start, end, case.M_cap)
    rows = np.flatnonzero(live)
    q, b = M.act_quant_rows_g128(case.gateup[rows], case.I, clamp)
    assert np.array_equal(hq[rows], q), "FP8 codes differ"
    assert np.array_equal(hs[:, rows].T, M.pack_g128_words(b)), "packed scales differ"
    assert np.all(hq[~live] == BYTE_SENT) and np.all(hs[:, ~live] == WORD_SENT)


@pytest.mark.parametrize("gemm,K,N", [(1, 640, 384), (2, 2048, 256), (1, 128, 256)])
def test_grouped_gemm_g128(ops, gemm, K, N):
    """Edge layouts (empty, exact-128, 129-row, single-row, multi-chunk
    experts); K = 640 ends on a word with one group, K = 128 has one k-step."""
    say(f"grouped gemm{gemm} g128 K={K} N={N}")
    rng = np.random.default_rng(K + N + gemm)
    counts, A = [0, 128, 129, 1, 300, 0, 17], 128
    E = len(counts)
    start, end = M.endpoints(np.array(counts, np.int64), A)
    M_cap = M.align_up(int(end[-1]), A)
    xq = rng.integers(0, 256, size=(M_cap, K), dtype=np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x3C
    b128 = rng.integers(120, 131, size=(M_cap, K // 128), dtype=np.uint8)
    xs = np.ascontiguousarray(M.pack_g128_words(b128).T)
    w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ws = rng.integers(120, 131, size=(E, N, K // 32), dtype=np.uint8)
    wp, sp = ops.moe_pack_mx_weights(dev(w), dev(ws))
    out = torch.full((M_cap, N), BF16_SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ends_d = dev(end.astype(np.int32))
    if gemm == 1:
        assert N % 2 == 0
        ops.moe_grouped_gemm1(dev(xq), dev(xs), ends_d, A, wp, sp, out, group=128)
    else:
        ops.moe_grouped_gemm2(dev(xq), dev(xs), ends_d, A, wp, sp, out, group=128)
    got = host(out)
    live = M.live_row_mask(start, end, M_cap)
    for e in range(E):
        rows = np.arange(start[e], end[e])
        if rows.size == 0:
            continue
        ab = M.expand_g128_bytes(b128[rows])
        _, exact, tsum = M.mx_gemm(xq[rows], ab, w[e], ws[e])
        bm = M.block_max_bound(xq[rows], ab, w[e], ws[e])
        ok, _, _ = gemm_within_bound(got[rows], exact, tsum, K, bm)
        assert ok.all(), f"expert {e}: {np.count_nonzero(~ok)} of {ok.size} outside bound"
    assert np.all(got[~live] == BF16_SENT)


@pytest.mark.parametrize("I,clamp,H", [(128, 0.0, 256), (640, 6.0, 640), (384, 0.0, 768)])
def test_gemm1_act_quant_fused_g128_equals_two_calls(ops, I, clamp, H):
    """moe_grouped_gemm1_act_quant_g128 against moe_grouped_gemm1(group 128)
    then moe_act_quant_liverows(group 128), byte for byte, on the edge
    layouts; I = 640 ends on a word with one group and three zero bytes; the
    two-call path itself against the oracle's group-128 act-quant."""
    say(f"fused gemm1+act-quant g128 I={I} clamp={clamp} H={H}")
    rng = np.random.default_rng(I + H)
    counts, A = [0, 128, 129, 1, 300, 0, 17], 128
    E = len(counts)
    start, end = M.endpoints(np.array(counts, np.int64), A)
    M_cap = M.align_up(int(end[-1]), A)
    xq = rng.integers(0, 256, size=(M_cap, H), dtype=np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x3C
    b128 = rng.integers(118, 128, size=(M_cap, H // 128), dtype=np.uint8)
    xs = np.ascontiguousarray(M.pack_g128_words(b128).T)
    w13 = rng.integers(0, 256, size=(E, 2 * I, H // 2), dtype=np.uint8)
    s13 = rng.integers(118, 128, size=(E, 2 * I, H // 32), dtype=np.uint8)
    ends_d = dev(end.astype(np.int32))
    wp, sp = ops.moe_pack_mx_weights(dev(w13), dev(s13))
    gp, gs = ops.moe_pack_mx_weights_gateup(dev(w13), dev(s13))
    gateup = torch.full((M_cap, 2 * I), BF16_SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    outs = []
    for fused in (False, True):
        hq = torch.full((M_cap, I), BYTE_SENT, dtype=torch.uint8, device="cuda")
        hs = torch.full((_words(I), M_cap), int(WORD_SENT), dtype=torch.int32, device="cuda")
        if fused:
            ops.moe_grouped_gemm1_act_quant(dev(xq), dev(xs), ends_d, A, gp, gs, clamp, hq, hs, group=128)
        else:
            ops.moe_grouped_gemm1(dev(xq), dev(xs), ends_d, A, wp, sp, gateup, group=128)
            ops.moe_act_quant_liverows(gateup, ends_d, A, clamp, hq, hs, group=128)
        outs.append((host(hq), host(hs)))
    (hq0, hs0), (hq1, hs1) = outs
    assert np.array_equal(hq0, hq1), "FP8 codes differ"
    assert np.array_equal(hs0, hs1), "packed scales differ"
    live = M.live_row_mask(start, end, M_cap)
    assert np.all(hq1[~live] == BYTE_SENT) and np.all(hs1[:, ~live] == WORD_SENT)
    rows = np.flatnonzero(live)
    q, b = M.act_quant_rows_g128(host(gateup)[rows], I, clamp)
    assert np.array_equal(hq0[rows], q) and np.array_equal(hs0[:, rows].T, M.pack_g128_words(b))


def test_prefill_layer_fused_g128_equals_two_calls(ops):
    """The prefill EP-share GEMM1 at full size: fused group-128 output equals
    the two-call group-128 output byte for byte."""
    c = W.prefill()
    w = c.weights
    ids, _ = M.route_softmax(c.logits, c.k)
    say("fused gemm1+act-quant g128, prefill EP share")
    buf = ops.alloc_grouped(c.T, c.k, c.E_local, c.M_cap, c.H, c.I, fill=True, group=128)
    xs = buf.xs
    ops.moe_scatter_endpoints(dev(ids), 0, c.E_local, c.A, dev_bf16(c.x), buf.expert_ends, buf.route_row,
                              buf.xq, xs, buf.workspace, group=128)
    wp, sp = ops.moe_pack_mx_weights(dev(w.w13), dev(w.s13))
    gp, gs = ops.moe_pack_mx_weights_gateup(dev(w.w13), dev(w.s13))
    outs = []
    for fused in (False, True):
        hq = torch.full((c.M_cap, c.I), BYTE_SENT, dtype=torch.uint8, device="cuda")
        hs = torch.full((_words(c.I), c.M_cap), int(WORD_SENT), dtype=torch.int32, device="cuda")
        if fused:
            ops.moe_grouped_gemm1_act_quant(buf.xq, xs, buf.expert_ends, c.A, gp, gs, c.clamp, hq, hs,
                                            group=128)
        else:
            ops.moe_grouped_gemm1(buf.xq, xs, buf.expert_ends, c.A, wp, sp, buf.gateup, group=128)
            ops.moe_act_quant_liverows(buf.gateup, buf.expert_ends, c.A, c.clamp, hq, hs, group=128)
        outs.append((host(hq), host(hs)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
