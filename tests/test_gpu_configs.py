"""GPU parity at the exact workload shapes, end to end and stage by stage:

* the prefill EP-share layer (the 4,096-token group of an EP8 layer, top-6
  of 256, this GPU's 32 experts, H=4,096, I=2,048): every live row of both
  GEMMs within the derived bound, act-quant and combine bit-exact, the final
  output of all 4,096 tokens against the oracle, and two runs bitwise equal;
  the same layer at 64 and 1,024 tokens per GPU end to end;
* the sparse decode layer (32 resident experts, H=2,880, top-4) at
  T = 1, 2, 4, 8 with FP8 and MXFP4 weights: each GEMV stage within a bound
  derived from the oracle's sum of |terms|, the GLU within one bf16 step,
  combine bit-exact, the output against the oracle, two runs bitwise equal.

Every call goes through the C ABI (``ops`` only marshals)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import moe as M
from tests.gpu_helpers import (BF16_SENT, BYTE_SENT, dev, dev_bf16, end_to_end_ok,
                               gemm_within_bound, host, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import mixture_experts_ffn_scatter_amd as pkg
    pkg.lib()
    return pkg.ops


def _segments(starts, ends):
    return [np.arange(int(s), int(e)) for s, e in zip(starts, ends)]


# ------------------------------------------------------- prefill EP share

def test_ep_share_layer_end_to_end(ops):
    c = W.prefill()
    w = c.weights
    ids, wts = M.route_softmax(c.logits, c.k)
    say("EP-share layer: oracle (expert-major chain, all 4,096 tokens)")
    ref = M.prefill_expert_major(c.x, ids, wts, 0, c.E_local, c.A, c.I, w.w13, w.s13, w.w2,
                                 w.s2, workers=8)
    sc = ref.scatter
    segs = _segments(sc.start, sc.end)
    live = M.live_row_mask(sc.start, sc.end, c.M_cap)

    say("EP-share layer: fused chain twice (the timed form)")
    x, ids_d, wts_d = dev_bf16(c.x), dev(ids), dev(wts)
    gp = ops.moe_pack_mx_weights_gateup(dev(w.w13), dev(w.s13))
    w2p = ops.moe_pack_mx_weights(dev(w.w2), dev(w.s2))
    runs = []
    for _ in range(2):
        buf = ops.alloc_grouped(c.T, c.k, c.E_local, c.M_cap, c.H, c.I, fill=True)
        y = ops.moe_ffn_prefill_fused(x, ids_d, wts_d, 0, c.A, *gp, *w2p, buf)
        runs.append(dict(out=host(y), hq=host(buf.hq), hs=host(buf.hs), down=host(buf.down),
                         xq=host(buf.xq), xs=host(buf.xs), ends=host(buf.expert_ends),
                         rr=host(buf.route_row)))
        del buf
    for key in runs[0]:
        assert np.array_equal(runs[0][key], runs[1][key]), f"run-to-run difference in {key}"
    r = runs[0]
    assert np.array_equal(r["ends"], sc.end.astype(np.int32))
    assert np.array_equal(r["rr"], sc.route_row)

    say("EP-share layer: scatter bytes, padding untouched")
    lr = sc.local_routes
    assert np.array_equal(r["xq"][sc.route_row[lr]], ref.xq)
    assert np.array_equal(r["xs"][:, sc.route_row[lr]].T, F.pack_ue8m0_words(ref.xb))
    assert np.all(r["xq"][~live] == BYTE_SENT) and np.all(r["hq"][~live] == BYTE_SENT)
    assert np.all(r["down"][~live] == BF16_SENT)

    say("EP-share layer: GEMM1 (two-call form) on every live row")
    w13p = ops.moe_pack_mx_weights(dev(w.w13), dev(w.s13))
    buf = ops.alloc_grouped(c.T, c.k, c.E_local, c.M_cap, c.H, c.I, fill=True)
    ops.moe_scatter_endpoints(ids_d, 0, c.E_local, c.A, x, buf.expert_ends, buf.route_row,
                              buf.xq, buf.xs, buf.workspace)
    ops.moe_grouped_gemm1(buf.xq, buf.xs, buf.expert_ends, c.A, *w13p, buf.gateup)
    ops.moe_act_quant_liverows(buf.gateup, buf.expert_ends, c.A, 0.0, buf.hq, buf.hs)
    gu, hq2, hs2 = host(buf.gateup), host(buf.hq), host(buf.hs)
    del buf
    assert np.all(gu[~live] == BF16_SENT)
    # the oracle's rows are in route order; the layout row of each is route_row
    row_of = sc.route_row[lr]
    n_checked = 0
    for e, rows in enumerate(segs):
        if rows.size == 0:
            continue
        sel = np.flatnonzero(sc.local_expert == e)      # oracle rows of expert e, in layout order
        assert np.array_equal(row_of[sel], rows)
        bm = M.block_max_bound(ref.xq[sel], ref.xb[sel], w.w13[e], w.s13[e])
        ok, _, _ = gemm_within_bound(gu[rows], ref.gateup_exact[sel], ref.gateup_tsum[sel], c.H, bm)
        assert ok.all(), f"gemm1 expert {e}: {np.count_nonzero(~ok)} of {ok.size} outside the bound"
        n_checked += rows.size
    assert n_checked == int(live.sum())

    say("EP-share layer: act-quant bit-exact on every live row; fused == two-call")
    rows = np.flatnonzero(live)
    q, b = M.act_quant_rows(gu[rows], c.I)
    assert np.array_equal(hq2[rows], q) and np.array_equal(hs2[:, rows].T, F.pack_ue8m0_words(b))
    assert np.array_equal(hq2, r["hq"]) and np.array_equal(hs2, r["hs"])

    say("EP-share layer: GEMM2 on every live row (from the GPU's hq)")
    hb = F.unpack_ue8m0_words(r["hs"].T)          # [M_cap, I/32]

    def gemm2_expert(e):
        rows_e = segs[e]
        if rows_e.size == 0:
            return 0
        _, exact, tsum = M.mx_gemm(r["hq"][rows_e], hb[rows_e], w.w2[e], w.s2[e])
        bm = M.block_max_bound(r["hq"][rows_e], hb[rows_e], w.w2[e], w.s2[e])
        ok, _, _ = gemm_within_bound(r["down"][rows_e], exact, tsum, c.I, bm)
        return int(np.count_nonzero(~ok))

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(8) as ex:
        bad = list(ex.map(gemm2_expert, range(c.E_local)))
    assert sum(bad) == 0, f"gemm2 rows outside the bound per expert: {bad}"

    say("EP-share layer: combine bit-exact, output of all 4,096 tokens vs the oracle")
    rows_f32 = F.bf16_to_f32(r["down"]).astype(np.float32)
    rows_f32[~live] = 0.0
    assert np.array_equal(r["out"], M.combine(rows_f32, r["rr"], wts, 1.0))
    ok, mx, mean = end_to_end_ok(r["out"], ref.out)
    say(f"  max |d| / max |ref| = {mx:.3e}, mean |d| / rms(ref) = {mean:.3e}")
    assert ok, (mx, mean)
    no_local = ~np.any((ids >= 0) & (ids < c.E_local), axis=1)
    assert np.all(r["out"][no_local] == 0)


@pytest.mark.parametrize("tokens_per_gpu", [64, 1024])
def test_ep_share_layer_token_counts(ops, tokens_per_gpu):
    """The same EP-share layer at 64 and 1,024 tokens per GPU (512- and
    8,192-token groups): thin one-chunk experts, and many-chunk experts that
    the schedule spreads over XCDs. Endpoints and route rows exact, combine
    bit-exact from the GPU's down rows, the output against the oracle, and
    tokens with no local route exactly zero."""
    c = W.prefill(tokens_per_gpu=tokens_per_gpu)
    w = c.weights
    ids, wts = M.route_softmax(c.logits, c.k)
    say(f"EP-share layer at {tokens_per_gpu} tokens/GPU: oracle")
    ref = M.prefill_expert_major(c.x, ids, wts, 0, c.E_local, c.A, c.I, w.w13, w.s13, w.w2,
                                 w.s2, workers=8)
    sc = ref.scatter
    live = M.live_row_mask(sc.start, sc.end, c.M_cap)
    say(f"EP-share layer at {tokens_per_gpu} tokens/GPU: fused chain, T={c.T} M_cap={c.M_cap}")
    gp = ops.moe_pack_mx_weights_gateup(dev(w.w13), dev(w.s13))
    w2p = ops.moe_pack_mx_weights(dev(w.w2), dev(w.s2))
    buf = ops.alloc_grouped(c.T, c.k, c.E_local, c.M_cap, c.H, c.I, fill=True)
    y = ops.moe_ffn_prefill_fused(dev_bf16(c.x), dev(ids), dev(wts), 0, c.A, *gp, *w2p, buf)
    out, down, rr = host(y), host(buf.down), host(buf.route_row)
    assert np.array_equal(host(buf.expert_ends), sc.end.astype(np.int32))
    assert np.array_equal(rr, sc.route_row)
    assert np.all(down[~live] == BF16_SENT)
    rows_f32 = F.bf16_to_f32(down).astype(np.float32)
    rows_f32[~live] = 0.0
    assert np.array_equal(out, M.combine(rows_f32, rr, wts, 1.0))
    ok, mx, mean = end_to_end_ok(out, ref.out)
    say(f"  max |d| / max |ref| = {mx:.3e}, mean |d| / rms(ref) = {mean:.3e}")
    assert ok, (mx, mean)
    no_local = ~np.any((ids >= 0) & (ids < c.E_local), axis=1)
    assert np.all(out[no_local] == 0)


# ------------------------------------------------------------ sparse decode

def _gemv_ok(got_bits, want_bits, tsum):
    """A GEMV output against the oracle's. The oracle rounds the exact sum
    once; the kernel sums each row along a tree of at most 80 fp32 additions
    (16 two-term dot steps per 32-weight chunk, up to 2 chunks per thread, 6
    wave levels, 4 waves), so the two fp32 values before the epilogue differ
    by at most 2^-17 * sum|t| (2^-24 per addition, with margin; the fp32
    epilogue roundings are of the same order and inside that margin). Each
    side then rounds to bf16 on its own, which moves it by at most half a
    bf16 step, i.e. 2^-8 of its magnitude: the two outputs may sit a whole
    step apart when the fp32 values straddle a rounding boundary."""
    g = F.bf16_to_f32(got_bits).astype(np.float64)
    o = F.bf16_to_f32(want_bits).astype(np.float64)
    bound = 2.0 ** -8 * (np.abs(g) + np.abs(o)) + 2.0 ** -17 * tsum + 1e-30
    ok = np.abs(g - o) <= bound
    if not ok.all():
        i = int(np.argmax(np.abs(g - o) - bound))
        say(f"  worst: got {g[i]!r} want {o[i]!r} sum|t| {tsum[i]!r} bound {bound[i]!r}")
    return ok


def _bf16_step(v):
    """The spacing of bf16 values at |v| (2^(e-7) for |v| in [2^e, 2^(e+1)))."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def _decode_weights(c):
    dw = [dev(c.w_gu), dev(c.s_gu), dev_bf16(c.b_gu), dev(c.w_d), dev(c.s_d), dev_bf16(c.b_d)]
    return dw


@pytest.mark.parametrize("wfmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_decode_exact_config(ops, wfmt, T):
    say(f"decode 32 experts H=2880 {wfmt} T={T}: inputs")
    c = W.decode(T=T, wfmt=wfmt)
    assert c.E == 32 and c.H == 2880 and c.k == 4 and c.w_gu.shape[0] == 32
    ids, wts = M.route_softmax(c.logits, c.k)
    ref = M.decode_chain(c, 0, 32, ids=ids, weights=wts)
    dw = _decode_weights(c)
    x, ids_d, wts_d = dev_bf16(c.x), dev(ids), dev(wts)
    gemv = M.gemv_fp8 if wfmt == "fp8" else M.gemv_mxfp4
    H = c.H

    say("  chain twice")
    runs = []
    for _ in range(2):
        buf = ops.alloc_decode(T, c.k, H, fill=True)
        y = ops.moe_ffn_decode(x, ids_d, wts_d, 0, 32, wfmt, *dw, buf)
        runs.append((host(y), host(buf.act), host(buf.down), host(buf.slot_row)))
    for a, b in zip(*runs):
        assert np.array_equal(a, b)
    out, act, down, slot_row = runs[0]
    assert np.array_equal(slot_row, ref.slot_row)

    say("  gate_up GEMV alone (no GLU) within the derived bound")
    gu = torch.full((T * c.k, c.N_gu), BF16_SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ops.moe_sparse_gemv(x, False, ids_d, 0, 32, wfmt, dw[0], dw[1], dw[2], gu, None, glu=False)
    gu = host(gu)
    for (t, s), want in ref.gu.items():
        e = int(ids[t, s])
        _, tsum = gemv(c.x[t:t + 1], c.w_gu[e], c.s_gu[e], c.b_gu[e])
        ok = _gemv_ok(gu[t * c.k + s], want, tsum[0])
        assert ok.all(), f"gate_up slot ({t},{s}): {np.count_nonzero(~ok)} outside the bound"

    say("  fused GLU within one bf16 step of the oracle's GLU of the GPU's gate_up")
    for (t, s) in ref.act:
        q = t * c.k + s
        a_ref = F.bf16_to_f32(M.glu(gu[q, :H], gu[q, H:], c.glu_alpha, c.glu_beta,
                                    c.glu_limit)).astype(np.float64)
        a_got = F.bf16_to_f32(act[q]).astype(np.float64)
        assert np.all(np.abs(a_got - a_ref) <= _bf16_step(a_ref))

    say("  GLU on load: down over the gate_up rows equals down over the fused GLU's rows")
    dn2 = torch.full((T * c.k, H), BF16_SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    gu_d = torch.from_numpy(gu.view(np.int16)).cuda().view(torch.bfloat16)
    ops.moe_sparse_gemv(gu_d, True, ids_d, 0, 32, wfmt, dw[3], dw[4], dw[5], dn2, None,
                        glu_on_load=True)
    assert np.array_equal(host(dn2), down)

    say("  down GEMV from the GPU's activations within the derived bound")
    for (t, s) in ref.down:
        e, q = int(ids[t, s]), t * c.k + s
        d, tsum = gemv(act[q:q + 1], c.w_d[e], c.s_d[e], c.b_d[e])
        ok = _gemv_ok(down[q], d[0], tsum[0])
        assert ok.all(), f"down slot ({t},{s}): {np.count_nonzero(~ok)} outside the bound"

    say("  combine bit-exact, output vs the oracle")
    assert np.array_equal(out, M.combine(F.bf16_to_f32(down), slot_row, wts, 1.0))
    ok, mx, mean = end_to_end_ok(out, ref.out)
    say(f"  max |d| / max |ref| = {mx:.3e}, mean |d| / rms(ref) = {mean:.3e}")
    assert ok, (mx, mean)
