"""GPU parity of the prefill path (route, scatter, GEMM1, act-quant, GEMM2,
combine) against the CPU oracle, through the C ABI.

Each stage is fed the GPU's own input to that stage (which earlier tests
pin bit-exactly), so integer and byte outputs must match the oracle bit for
bit and float GEMM outputs must sit within the accumulation bound. Padding
of every grouped buffer is seeded with sentinels that must survive."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import moe as M
from tests.gpu_helpers import (BF16_SENT, BYTE_SENT, WORD_SENT, actquant_case, dev, dev_bf16, end_to_end_ok,
                               gemm_within_bound, host, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import mixture_experts_ffn_scatter_amd as pkg
    pkg.lib()
    return pkg.ops


# ------------------------------------------------------------------ routing

@pytest.mark.parametrize("case", ["tiny", "ties", "prefill-own", "prefill-group", "decode", "large"])
def test_route_ids_bitexact(ops, case):
    say(f"route {case}")
    bias = None
    if case == "tiny":
        c = W.tiny(); logits, k = c.logits, c.k
    elif case == "ties":
        # few distinct values, signed zeros and -inf: the order falls to the index
        rng = np.random.default_rng(11)
        vals = np.array([0.0, -0.0, 1.0, -1.0, 0.5], dtype=np.float32)
        logits, k = vals[rng.integers(0, len(vals), size=(300, 160))], 8
        logits[::7, :3] = -np.inf
        logits[1::7, :] = -0.0
        logits[1::7, 5::9] = 0.0
    elif case == "prefill-own":
        c = W.prefill(with_weights=False); logits, k = c.logits[:512], c.k
    elif case == "prefill-group":
        c = W.prefill(with_weights=False); logits, k = c.logits, c.k
    elif case == "decode":
        c = W.decode(T=8, H=64, experts=1); logits, k = c.logits, c.k
    else:
        c = W.large(with_weights=False); logits, k, bias = c.logits, c.k, c.bias
    if bias is None:
        ids_o, w_o = M.route_softmax(logits, k)
        ids, w = ops.moe_route(dev(logits), k, "softmax")
    else:
        ids_o, w_o = M.route_sigmoid_bias(logits, bias, k)
        ids, w = ops.moe_route(dev(logits), k, "sigmoid_bias", dev(bias))
    ids, w = host(ids), host(w)
    assert np.array_equal(ids, ids_o)
    assert np.allclose(w, w_o, rtol=4 * 2.0 ** -23, atol=0)


# ------------------------------------------------------------------ scatter

def _run_scatter(ops, ids, x_bits, expert_start, E_local, A, M_cap):
    T, k = ids.shape
    H = x_bits.shape[1]
    ends = torch.full((E_local,), -7, dtype=torch.int32, device="cuda")
    rr = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    xq = torch.full((M_cap, H), BYTE_SENT, dtype=torch.uint8, device="cuda")
    xs = torch.full((H // 128, M_cap), int(WORD_SENT), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(ops.moe_scatter_workspace_bytes(T, k, E_local), 1), dtype=torch.uint8,
                     device="cuda")
    ops.moe_scatter_endpoints(dev(ids.astype(np.int32)), expert_start, E_local, A,
                              dev_bf16(x_bits), ends, rr, xq, xs, ws)
    return host(ends), host(rr), host(xq), host(xs)


def _check_scatter(ids, x_bits, expert_start, E_local, A, M_cap, got):
    ends, rr, xq, xs = got
    sc = M.scatter_routes(ids, expert_start, E_local, A)
    assert np.array_equal(ends, sc.end.astype(np.int32))
    assert np.array_equal(rr, sc.route_row)
    k = ids.shape[1]
    rows = sc.route_row[sc.local_routes]
    q, b = M.quant_rows(x_bits[sc.local_routes // k])
    assert np.array_equal(xq[rows], q)
    words = F.pack_ue8m0_words(b) if b.size else np.zeros((0, x_bits.shape[1] // 128), np.int32)
    assert np.array_equal(xs[:, rows].T, words)
    live = M.live_row_mask(sc.start, sc.end, M_cap)
    assert np.all(xq[~live] == BYTE_SENT)
    assert np.all(xs[:, ~live] == WORD_SENT)


def test_scatter_tiny(ops):
    say("scatter tiny")
    c = W.tiny()
    ids, _ = M.route_softmax(c.logits, c.k)
    got = _run_scatter(ops, ids, c.x, 0, c.E, c.A, c.M_cap)
    _check_scatter(ids, c.x, 0, c.E, c.A, c.M_cap, got)


def test_scatter_window_negative_ids_small_alignment(ops):
    say("scatter window/-1/A=16")
    c = W.tiny(seed=77, T=40)
    ids, _ = M.route_softmax(c.logits, c.k)
    ids = ids.copy()
    ids[3, 1] = -1
    ids[7, 0] = -1
    M_cap = W.capacity(40, 2, 4, 16)
    got = _run_scatter(ops, ids, c.x, 2, 4, 16, M_cap)
    _check_scatter(ids, c.x, 2, 4, 16, M_cap, got)


def test_scatter_all_nonlocal_and_duplicate_ids(ops):
    say("scatter all-nonlocal / duplicates")
    c = W.tiny(seed=5, T=20)
    ids = np.full((20, 2), 50, np.int32)
    M_cap = W.capacity(20, 2, 8, 128)
    got = _run_scatter(ops, ids, c.x, 0, 8, 128, M_cap)
    _check_scatter(ids, c.x, 0, 8, 128, M_cap, got)
    ids = np.stack([np.arange(20) % 3, np.arange(20) % 3], axis=1).astype(np.int32)  # both slots equal
    got = _run_scatter(ops, ids, c.x, 0, 8, 128, M_cap)
    _check_scatter(ids, c.x, 0, 8, 128, M_cap, got)


def test_scatter_fp8_rounding_edges(ops):
    """Inputs built so that v / 2^(b-127) lands on E4M3 midpoints, on codes,
    in the subnormal range and on zeros, to pin the hardware conversion."""
    say("scatter fp8 rounding edges")
    rng = np.random.default_rng(21)
    T, H = 48, 512
    pos = F.E4M3_VALUES[:127]
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.empty((T, H), np.float64)
    for t in range(T):
        for g in range(H // 32):
            j = int(rng.integers(-30, 20))
            sf = 2.0 ** j
            vals = rng.choice(np.concatenate([mids, pos, mids[:16] * 1.0078125]), 32)
            vals *= rng.choice([-1.0, 1.0], 32)
            vals[int(rng.integers(0, 32))] = 448.0 * rng.choice([-1, 1])
            if g % 5 == 0:
                vals[:] = 0.0
            x[t, g * 32:(g + 1) * 32] = vals * sf
    xb = F.round_to_bf16(x)
    ids = np.stack([np.arange(T) % 4, 4 + np.arange(T) % 3], axis=1).astype(np.int32)
    M_cap = W.capacity(T, 2, 8, 128)
    got = _run_scatter(ops, ids, xb, 0, 8, 128, M_cap)
    _check_scatter(ids, xb, 0, 8, 128, M_cap, got)


def test_scatter_scale_byte_edges(ops):
    """Group maxima at 448 * 2^j and the bf16 values just above and below it,
    for j over the whole bf16 range (subnormal quotients included), plus
    bf16 subnormal and all-zero groups: the UE8M0 byte decision at every
    power-of-two boundary."""
    say("scatter scale-byte edges")
    rng = np.random.default_rng(22)
    T, H = 64, 1024
    G = H // 32
    js = np.arange(-141, 120)
    x = np.empty((T, H), np.float64)
    for t in range(T):
        for g in range(G):
            j = int(js[(t * G + g) % js.size])
            top = 448.0 * 2.0 ** j
            kind = (t * G + g) // js.size % 4
            if kind == 1:
                top *= 1.0 + 2.0 ** -7        # next bf16 above
            elif kind == 2:
                top *= 1.0 - 2.0 ** -8        # next bf16 below
            elif kind == 3:
                top = 2.0 ** -133 * int(rng.integers(0, 128))   # bf16 subnormals (and zero)
            vals = rng.uniform(-1.0, 1.0, 32) * top
            vals[int(rng.integers(0, 32))] = top * rng.choice([-1.0, 1.0])
            x[t, g * 32:(g + 1) * 32] = vals
    xb = F.round_to_bf16(x)
    assert np.all(np.isfinite(F.bf16_to_f32(xb)))
    ids = np.stack([np.arange(T) % 5, 5 + np.arange(T) % 3], axis=1).astype(np.int32)
    M_cap = W.capacity(T, 2, 8, 128)
    got = _run_scatter(ops, ids, xb, 0, 8, 128, M_cap)
    _check_scatter(ids, xb, 0, 8, 128, M_cap, got)


@pytest.mark.parametrize("T,k,E,start,E_local", [(2048, 16, 896, 0, 896), (4096, 8, 1200, 100, 1024)])
def test_scatter_long_token_blocks(ops, T, k, E, start, E_local):
    """Many routes per token block (more than 512 earlier routes for a
    token's rank), and a block-by-expert table too large for 64-token blocks
    (4096 tokens x 1024 local experts), with skewed ids, -1 slots and ids
    outside the window."""
    say(f"scatter T={T} k={k} E={E} window [{start}, {start + E_local})")
    rng = np.random.default_rng(T + k)
    # Gumbel-top-k over Zipf(1.0) popularity on a shuffled expert order
    logp = -np.log(1.0 + rng.permutation(E))
    keys = logp[None, :] + rng.gumbel(size=(T, E))
    ids = np.argsort(-keys, axis=1)[:, :k].astype(np.int32)
    ids[rng.random((T, k)) < 0.02] = -1
    H, A = 128, 128
    x = F.round_to_bf16(rng.standard_normal((T, H)))
    M_cap = W.capacity(T, k, E_local, A)
    got = _run_scatter(ops, ids, x, start, E_local, A, M_cap)
    _check_scatter(ids, x, start, E_local, A, M_cap, got)


def test_scatter_prefill_group_full_size(ops):
    say("scatter prefill EP group 4096x6 -> 32 local experts")
    c = W.prefill(with_weights=False)
    ids, _ = M.route_softmax(c.logits, c.k)
    got = _run_scatter(ops, ids, c.x, 0, c.E_local, c.A, c.M_cap)
    _check_scatter(ids, c.x, 0, c.E_local, c.A, c.M_cap, got)


# ---------------------------------------------------------------- act-quant

def _run_act(ops, case, clamp=0.0):
    start, end = M.endpoints(case.counts, case.A)
    hq = torch.full((case.M_cap, case.I), BYTE_SENT, dtype=torch.uint8, device="cuda")
    hs = torch.full((case.I // 128, case.M_cap), int(WORD_SENT), dtype=torch.int32, device="cuda")
    ops.moe_act_quant_liverows(dev_bf16(case.gateup), dev(end.astype(np.int32)), case.A, clamp,
                               hq, hs)
    return start, end, host(hq), host(hs)


def _check_act(case, start, end, hq, hs, rows, clamp=0.0):
    q, b = M.act_quant_rows(case.gateup[rows], case.I, clamp)
    assert np.array_equal(hq[rows], q), "FP8 codes differ"
    assert np.array_equal(hs[:, rows].T, F.pack_ue8m0_words(b)), "packed scales differ"
    live = M.live_row_mask(start, end, case.M_cap)
    assert np.all(hq[~live] == BYTE_SENT)
    assert np.all(hs[:, ~live] == WORD_SENT)


def test_act_quant_liverows_3072_of_28672(ops):
    say("act-quant 3072 live of 28672")
    case = actquant_case()
    start, end, hq, hs = _run_act(ops, case)
    live = np.flatnonzero(M.live_row_mask(start, end, case.M_cap))
    assert live.size == 3072
    _check_act(case, start, end, hq, hs, live)


def test_act_quant_full_buffer_sampled(ops):
    say("act-quant full buffer 28672 rows")
    case = actquant_case(full=True)
    start, end, hq, hs = _run_act(ops, case)
    rows = np.sort(np.random.default_rng(3).choice(case.M_cap, 1024, replace=False))
    _check_act(case, start, end, hq, hs, rows)


def test_act_quant_clamp_small_I_odd_alignment(ops):
    say("act-quant clamp 25, I=384, A=8")
    rng = np.random.default_rng(9)
    counts = np.array([5, 0, 17, 1, 0, 9], np.int64)
    case = actquant_case(counts=counts, E_local=6, I=384, A=8, M_cap=64)
    # scale live rows so that the clamp engages on both sides
    live = M.live_row_mask(*M.endpoints(counts, 8), 64)
    g = F.bf16_to_f32(case.gateup).astype(np.float64) * 30.0
    g[~live] = np.nan
    case.gateup = F.round_to_bf16(g)
    start, end, hq, hs = _run_act(ops, case, clamp=25.0)
    _check_act(case, start, end, hq, hs, np.flatnonzero(live), clamp=25.0)


def test_act_quant_empty_and_all_empty(ops):
    say("act-quant all-empty")
    case = actquant_case(counts=np.zeros(4, np.int64), E_local=4, I=256, A=128, M_cap=512)
    start, end, hq, hs = _run_act(ops, case)
    assert np.all(hq == BYTE_SENT) and np.all(hs == WORD_SENT)


def _run_act_situ(ops, case):
    start, end = M.endpoints(case.counts, case.A)
    hq = torch.full((case.M_cap, case.I), BYTE_SENT, dtype=torch.uint8, device="cuda")
    hs = torch.full((case.I // 128, case.M_cap), int(WORD_SENT), dtype=torch.int32, device="cuda")
    ops.moe_act_quant_liverows_situ(dev_bf16(case.gateup), dev(end.astype(np.int32)), case.A, hq, hs)
    return start, end, host(hq), host(hs)


def _check_act_situ(case, start, end, hq, hs, rows):
    q, b = M.act_quant_rows_situ(case.gateup[rows], case.I)
    assert np.array_equal(hq[rows], q), "FP8 codes differ"
    assert np.array_equal(hs[:, rows].T, F.pack_ue8m0_words(b)), "packed scales differ"
    live = M.live_row_mask(start, end, case.M_cap)
    assert np.all(hq[~live] == BYTE_SENT)
    assert np.all(hs[:, ~live] == WORD_SENT)


def test_act_quant_situ_liverows_3072_of_28672(ops):
    """SiTU (Kimi-K3's 4 / 25) on the act-quant layout: bytes equal the
    oracle's on every live row, padding (NaN-filled) untouched."""
    say("act-quant SiTU 3072 live of 28672")
    case = actquant_case()
    start, end, hq, hs = _run_act_situ(ops, case)
    live = np.flatnonzero(M.live_row_mask(start, end, case.M_cap))
    _check_act_situ(case, start, end, hq, hs, live)


@pytest.mark.parametrize("side", ["gate", "up"])
def test_act_quant_situ_every_bf16(ops, side):
    """Every finite bf16 value as the gate (up = 1) or as the up input
    (gate = 1), sorted so that each 32-group holds neighbouring magnitudes:
    the codes then follow each function value, so every row of the tanh
    and sigmoid tables and both out-of-table rules are exercised."""
    say(f"act-quant SiTU every bf16 ({side})")
    b = np.arange(65536, dtype=np.uint32)
    b = b[((b >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    vals = np.sort(F.bf16_to_f32(b).astype(np.float64))
    I = 2048
    rows = -(-vals.size // I)
    x = np.zeros(rows * I)
    x[:vals.size] = vals
    one = np.ones(rows * I)
    g, u = (x, one) if side == "gate" else (one, x)
    gateup = np.concatenate([F.round_to_bf16(g.reshape(rows, I)), F.round_to_bf16(u.reshape(rows, I))], 1)
    counts = np.array([rows], np.int64)
    case = W.ActQuantCase("situ-every-bf16", 1, I, 128, 128, counts, gateup.astype(np.uint16))
    case.gateup = np.concatenate([gateup, np.full((128 - rows, 2 * I), 0x7FC1, np.uint16)])
    start, end, hq, hs = _run_act_situ(ops, case)
    _check_act_situ(case, start, end, hq, hs, np.arange(rows))


# -------------------------------------------------------------------- GEMMs

def _tiny_state(ops, c, clamp=0.0):
    ids, wts = M.route_softmax(c.logits, c.k)
    buf = ops.alloc_grouped(c.T, c.k, c.E, c.M_cap, c.H, c.I, fill=True)
    w = c.weights
    w13p, s13p = ops.moe_pack_mx_weights(dev(w.w13), dev(w.s13))
    w2p, s2p = ops.moe_pack_mx_weights(dev(w.w2), dev(w.s2))
    dw = dict(w13=w13p, s13=s13p, w2=w2p, s2=s2p)
    ops.moe_scatter_endpoints(dev(ids), 0, c.E, c.A, dev_bf16(c.x), buf.expert_ends, buf.route_row,
                              buf.xq, buf.xs, buf.workspace)
    return ids, wts, buf, dw


def _expert_rows(ends, A):
    prev = 0
    out = []
    for e in ends:
        s = ((prev + A - 1) // A) * A
        out.append(np.arange(s, e))
        prev = e
    return out


def test_gemm1_gemm2_combine_tiny_stagewise(ops):
    c = W.tiny()
    ids, wts, buf, dw = _tiny_state(ops, c)
    say("gemm1 tiny")
    ops.moe_grouped_gemm1(buf.xq, buf.xs, buf.expert_ends, c.A, dw["w13"], dw["s13"], buf.gateup)
    ends = host(buf.expert_ends)
    xq, xs, gu = host(buf.xq), host(buf.xs), host(buf.gateup)
    live = np.zeros(c.M_cap, bool)
    for e, rows in enumerate(_expert_rows(ends, c.A)):
        if rows.size == 0:
            continue
        live[rows] = True
        ab = F.unpack_ue8m0_words(xs[:, rows].T)
        _, exact, tsum = M.mx_gemm(xq[rows], ab, c.weights.w13[e], c.weights.s13[e])
        bm = M.block_max_bound(xq[rows], ab, c.weights.w13[e], c.weights.s13[e])
        ok, err, bound = gemm_within_bound(gu[rows], exact, tsum, c.H, bm)
        assert ok.all(), f"expert {e}: {np.count_nonzero(~ok)} of {ok.size} outside bound"
    assert np.all(gu[~live] == BF16_SENT)

    say("act-quant on GPU gateup")
    ops.moe_act_quant_liverows(buf.gateup, buf.expert_ends, c.A, 0.0, buf.hq, buf.hs)
    hq, hs = host(buf.hq), host(buf.hs)
    rows = np.flatnonzero(live)
    q, b = M.act_quant_rows(gu[rows], c.I)
    assert np.array_equal(hq[rows], q) and np.array_equal(hs[:, rows].T, F.pack_ue8m0_words(b))

    say("gemm2 tiny")
    ops.moe_grouped_gemm2(buf.hq, buf.hs, buf.expert_ends, c.A, dw["w2"], dw["s2"], buf.down)
    dn = host(buf.down)
    for e, rows_e in enumerate(_expert_rows(ends, c.A)):
        if rows_e.size == 0:
            continue
        hb_e = F.unpack_ue8m0_words(hs[:, rows_e].T)
        _, exact, tsum = M.mx_gemm(hq[rows_e], hb_e, c.weights.w2[e], c.weights.s2[e])
        bm = M.block_max_bound(hq[rows_e], hb_e, c.weights.w2[e], c.weights.s2[e])
        ok, _, _ = gemm_within_bound(dn[rows_e], exact, tsum, c.I, bm)
        assert ok.all(), f"expert {e}: {np.count_nonzero(~ok)} outside bound"
    assert np.all(dn[~live] == BF16_SENT)

    say("combine tiny")
    ops.moe_combine(buf.down, buf.route_row, dev(wts), 1.0, buf.out)
    out = host(buf.out)
    rows_f32 = F.bf16_to_f32(dn)
    ref = M.combine(rows_f32, host(buf.route_row), wts, 1.0)
    assert np.array_equal(out, ref)


def test_prefill_chain_tiny_end_to_end_and_deterministic(ops):
    c = W.tiny()
    ids, wts = M.route_softmax(c.logits, c.k)
    w = c.weights
    say("prefill chain tiny")
    ref = M.prefill_expert_major(c.x, ids, wts, 0, c.E, c.A, c.I, w.w13, w.s13, w.w2, w.s2)
    outs = []
    for _ in range(2):
        buf = ops.alloc_grouped(c.T, c.k, c.E, c.M_cap, c.H, c.I, fill=True)
        y = ops.moe_ffn_prefill(dev_bf16(c.x), dev(ids), dev(wts), 0, c.A,
                                *ops.moe_pack_mx_weights(dev(w.w13), dev(w.s13)),
                                *ops.moe_pack_mx_weights(dev(w.w2), dev(w.s2)), buf)
        outs.append(host(y))
    assert np.array_equal(outs[0], outs[1])
    ok, mx, mean = end_to_end_ok(outs[0], ref.out)
    assert ok, (mx, mean)


def test_prefill_chain_window_clamp_scale(ops):
    """Local window of 4 of 8 experts, -1 slots, A=16, clamp 6, routed scale 0.5."""
    c = W.tiny(seed=77, T=40)
    ids, wts = M.route_softmax(c.logits, c.k)
    ids = ids.copy()
    ids[3, 1] = -1
    w = c.weights
    E_local, es, A = 4, 2, 16
    M_cap = W.capacity(c.T, c.k, E_local, A)
    sl = slice(es, es + E_local)
    say("prefill chain window/clamp")
    ref = M.prefill_expert_major(c.x, ids, wts, es, E_local, A, c.I, w.w13[sl], w.s13[sl],
                                 w.w2[sl], w.s2[sl], clamp=6.0, routed_scale=0.5)
    buf = ops.alloc_grouped(c.T, c.k, E_local, M_cap, c.H, c.I, fill=True)
    y = ops.moe_ffn_prefill(dev_bf16(c.x), dev(ids), dev(wts), es, A,
                            *ops.moe_pack_mx_weights(dev(w.w13[sl]), dev(w.s13[sl])),
                            *ops.moe_pack_mx_weights(dev(w.w2[sl]), dev(w.s2[sl])), buf, clamp_limit=6.0,
                            routed_scale=0.5)
    ok, mx, mean = end_to_end_ok(host(y), ref.out)
    assert ok, (mx, mean)
    no_local = ~np.any((ids >= es) & (ids < es + E_local), axis=1)
    assert np.all(host(y)[no_local] == 0)


# ------------------------------------------------- weight prep + full size

def _expected_packing(w, s):
    """The documented packed layouts, built by plain indexing."""
    E, N, K2 = w.shape
    K = 2 * K2
    KS = K // 128
    lane = np.arange(64)
    wp = np.empty((E, N // 16, KS, 64, 16), np.uint8)
    sp = np.empty((E, KS, N // 64, 64, 4), np.uint8)
    for cb in range(N // 16):
        rows = 16 * cb + lane % 16
        for ks in range(KS):
            cols = 64 * ks + 16 * (lane // 16)
            wp[:, cb, ks] = w[:, rows[:, None], cols[:, None] + np.arange(16)[None, :]]
            # byte cb % 4 of lane l's word of column-block group cb // 4
            sp[:, ks, cb // 4, :, cb % 4] = s[:, rows, 4 * ks + lane // 16]
    return wp.reshape(E, N, K2), sp


def test_pack_mx_weights_bitexact(ops):
    """Load-time weight preparation is pure data movement into the documented
    fragment order (codes) and per-step, per-group lane words (scales)."""
    rng = np.random.default_rng(2024)
    for E, N, K in ((3, 192, 384), (1, 128, 128), (2, 256, 2048), (1, 64, 1152)):
        say(f"pack mx weights E={E} N={N} K={K}")
        w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
        s = rng.integers(0, 256, size=(E, N, K // 32), dtype=np.uint8)
        wp, sp = ops.moe_pack_mx_weights(dev(w), dev(s))
        ew, es = _expected_packing(w, s)
        assert np.array_equal(host(wp), ew)
        assert np.array_equal(host(sp), es)


def test_prefill_group_full_size_gemms_sampled(ops):
    """Full EP-share shapes (4096 group tokens x top-6 -> 32 local experts,
    H=4096, I=2048): GEMM1, act-quant, GEMM2 stage by stage on sampled rows
    (head and tail of the hottest, a middle and the coldest live expert)."""
    c = W.prefill()
    ids, wts = M.route_softmax(c.logits, c.k)
    w = c.weights
    say("full-size prefill GEMMs: scatter")
    buf = ops.alloc_grouped(c.T, c.k, c.E_local, c.M_cap, c.H, c.I, fill=True)
    ops.moe_scatter_endpoints(dev(ids), 0, c.E_local, c.A, dev_bf16(c.x), buf.expert_ends,
                              buf.route_row, buf.xq, buf.xs, buf.workspace)
    say("full-size prefill GEMMs: gemm1 / act-quant / gemm2")
    w13p, s13p = ops.moe_pack_mx_weights(dev(w.w13), dev(w.s13))
    w2p, s2p = ops.moe_pack_mx_weights(dev(w.w2), dev(w.s2))
    ops.moe_grouped_gemm1(buf.xq, buf.xs, buf.expert_ends, c.A, w13p, s13p, buf.gateup)
    ops.moe_act_quant_liverows(buf.gateup, buf.expert_ends, c.A, 0.0, buf.hq, buf.hs)
    ops.moe_grouped_gemm2(buf.hq, buf.hs, buf.expert_ends, c.A, w2p, s2p, buf.down)
    ends = host(buf.expert_ends)
    segs = _expert_rows(ends, c.A)
    counts = np.array([r.size for r in segs])
    live_e = np.flatnonzero(counts)
    order = live_e[np.argsort(counts[live_e], kind="stable")]
    picks = sorted({int(order[-1]), int(order[len(order) // 2]), int(order[0])})
    xq, xs, gu = host(buf.xq), host(buf.xs), host(buf.gateup)
    hq, hs, dn = host(buf.hq), host(buf.hs), host(buf.down)
    live = np.zeros(c.M_cap, bool)
    for rows in segs:
        live[rows] = True
    assert np.all(gu[~live] == BF16_SENT) and np.all(dn[~live] == BF16_SENT)
    for e in picks:
        rows = segs[e]
        rows = np.unique(np.concatenate([rows[:8], rows[-8:]]))
        say(f"  expert {e}: {segs[e].size} rows, checking {rows.size}")
        ab = F.unpack_ue8m0_words(xs[:, rows].T)
        _, exact, tsum = M.mx_gemm(xq[rows], ab, w.w13[e], w.s13[e])
        bm = M.block_max_bound(xq[rows], ab, w.w13[e], w.s13[e])
        ok, _, _ = gemm_within_bound(gu[rows], exact, tsum, c.H, bm)
        assert ok.all(), f"gemm1 expert {e}: {np.count_nonzero(~ok)} outside bound"
        q, b = M.act_quant_rows(gu[rows], c.I)
        assert np.array_equal(hq[rows], q)
        assert np.array_equal(hs[:, rows].T, F.pack_ue8m0_words(b))
        hb = F.unpack_ue8m0_words(hs[:, rows].T)
        _, exact, tsum = M.mx_gemm(hq[rows], hb, w.w2[e], w.s2[e])
        bm = M.block_max_bound(hq[rows], hb, w.w2[e], w.s2[e])
        ok, _, _ = gemm_within_bound(dn[rows], exact, tsum, c.I, bm)
        assert ok.all(), f"gemm2 expert {e}: {np.count_nonzero(~ok)} outside bound"


def test_large_e_full_size_chain_sampled(ops):
    """The large-expert-count layer at full size (2,048 tokens, top-16 sigmoid
    + bias over 896 resident experts, H=3,584, I=3,072, clamp 25): endpoints
    and permutation bit-exact; quantised x, GEMM1, act-quant and GEMM2 on
    sampled rows of the hottest, a middle and the coldest live expert; the
    fused GEMM1 + act-quant byte-identical to the two calls over the whole
    buffer; the fused chain run twice bitwise equal; combine bit-exact and
    64 tokens end to end against the oracle."""
    say("large-E full size: generating inputs (15.7 GB of weights)")
    c = W.large()
    w = c.weights
    ids, wts = M.route_sigmoid_bias(c.logits, c.bias, c.k)
    say("large-E full size: scatter")
    buf = ops.alloc_grouped(c.T, c.k, c.E_local, c.M_cap, c.H, c.I, fill=True)
    ops.moe_scatter_endpoints(dev(ids), 0, c.E_local, c.A, dev_bf16(c.x), buf.expert_ends,
                              buf.route_row, buf.xq, buf.xs, buf.workspace)
    sc = M.scatter_routes(ids, 0, c.E_local, c.A)
    ends = host(buf.expert_ends)
    rr = host(buf.route_row)
    assert np.array_equal(ends, sc.end.astype(np.int32))
    assert np.array_equal(rr, sc.route_row)
    say("large-E full size: packing weights, gemm1 / act-quant / gemm2")
    w13d, s13d = dev(w.w13), dev(w.s13)
    w13p, s13p = ops.moe_pack_mx_weights(w13d, s13d)
    w13g, s13g = ops.moe_pack_mx_weights_gateup(w13d, s13d)
    del w13d, s13d
    w2d, s2d = dev(w.w2), dev(w.s2)
    w2p, s2p = ops.moe_pack_mx_weights(w2d, s2d)
    del w2d, s2d
    ops.moe_grouped_gemm1(buf.xq, buf.xs, buf.expert_ends, c.A, w13p, s13p, buf.gateup)
    ops.moe_act_quant_liverows(buf.gateup, buf.expert_ends, c.A, c.clamp, buf.hq, buf.hs)
    ops.moe_grouped_gemm2(buf.hq, buf.hs, buf.expert_ends, c.A, w2p, s2p, buf.down)
    say("large-E full size: fused gemm1 + act-quant against the two calls")
    hq2 = torch.full_like(buf.hq, 0xA5)
    hs2 = torch.full_like(buf.hs, -1515870811)
    ops.moe_grouped_gemm1_act_quant(buf.xq, buf.xs, buf.expert_ends, c.A, w13g, s13g, c.clamp,
                                    hq2, hs2)
    assert torch.equal(hq2, buf.hq) and torch.equal(hs2, buf.hs)
    del hq2, hs2, w13g, s13g
    ops.moe_combine(buf.down, buf.route_row, dev(wts), 1.0, buf.out)
    torch.cuda.synchronize()
    segs = _expert_rows(ends, c.A)
    counts = np.array([r.size for r in segs])
    live_e = np.flatnonzero(counts)
    order = live_e[np.argsort(counts[live_e], kind="stable")]
    picks = sorted({int(order[-1]), int(order[len(order) // 2]), int(order[0])})
    xq, xs = host(buf.xq), host(buf.xs)
    gu, hq, hs, dn = host(buf.gateup), host(buf.hq), host(buf.hs), host(buf.down)
    live = np.zeros(c.M_cap, bool)
    for rows in segs:
        live[rows] = True
    assert np.all(gu[~live] == BF16_SENT) and np.all(dn[~live] == BF16_SENT)
    assert np.all(hq[~live] == BYTE_SENT) and np.all(xq[~live] == BYTE_SENT)
    for e in picks:
        rows = segs[e]
        rows = np.unique(np.concatenate([rows[:6], rows[-6:]]))
        say(f"  expert {e}: {segs[e].size} rows, checking {rows.size}")
        # quantised x of these rows: each row is the token its route came from
        src = np.array([int(np.flatnonzero(sc.route_row == r)[0]) // c.k for r in rows])
        q, b = M.quant_rows(c.x[src])
        assert np.array_equal(xq[rows], q)
        assert np.array_equal(xs[:, rows].T, F.pack_ue8m0_words(b))
        ab = F.unpack_ue8m0_words(xs[:, rows].T)
        _, exact, tsum = M.mx_gemm(xq[rows], ab, w.w13[e], w.s13[e])
        bm = M.block_max_bound(xq[rows], ab, w.w13[e], w.s13[e])
        ok, _, _ = gemm_within_bound(gu[rows], exact, tsum, c.H, bm)
        assert ok.all(), f"gemm1 expert {e}: {np.count_nonzero(~ok)} outside bound"
        q, b = M.act_quant_rows(gu[rows], c.I, c.clamp)
        assert np.array_equal(hq[rows], q)
        assert np.array_equal(hs[:, rows].T, F.pack_ue8m0_words(b))
        hb = F.unpack_ue8m0_words(hs[:, rows].T)
        _, exact, tsum = M.mx_gemm(hq[rows], hb, w.w2[e], w.s2[e])
        bm = M.block_max_bound(hq[rows], hb, w.w2[e], w.s2[e])
        ok, _, _ = gemm_within_bound(dn[rows], exact, tsum, c.I, bm)
        assert ok.all(), f"gemm2 expert {e}: {np.count_nonzero(~ok)} outside bound"
    say("large-E full size: the fused chain again, bitwise equal (determinism)")
    out = host(buf.out)
    w13g, s13g = ops.moe_pack_mx_weights_gateup(dev(w.w13), dev(w.s13))
    buf2 = ops.alloc_grouped(c.T, c.k, c.E_local, c.M_cap, c.H, c.I, fill=True)
    ops.moe_ffn_prefill_fused(dev_bf16(c.x), dev(ids), dev(wts), 0, c.A, w13g, s13g, w2p, s2p,
                              buf2, clamp_limit=c.clamp)
    y2 = ops.alloc_grouped(c.T, c.k, c.E_local, c.M_cap, c.H, c.I, fill=True)
    ops.moe_ffn_prefill_fused(dev_bf16(c.x), dev(ids), dev(wts), 0, c.A, w13g, s13g, w2p, s2p,
                              y2, clamp_limit=c.clamp)
    assert torch.equal(buf2.out.view(torch.int16), y2.out.view(torch.int16))
    assert torch.equal(buf2.down.view(torch.int16), y2.down.view(torch.int16))
    assert np.array_equal(host(buf2.out), out)      # and equal to the two-call chain above
    del buf2, y2, w13g, s13g

    # 64 tokens end to end: a greedy pick that keeps the set of experts they
    # route to small (so the oracle finishes in seconds), plus the first and
    # last token
    toks = [0, c.T - 1]
    used_e = set(ids[0].tolist()) | set(ids[c.T - 1].tolist())
    cand = set(range(1, c.T - 1))
    sets = [set(r.tolist()) for r in ids]
    while len(toks) < 64:
        t = max(cand, key=lambda u: (len(sets[u] & used_e), -u))
        toks.append(t)
        cand.remove(t)
        used_e |= sets[t]
    toks = np.array(sorted(toks))
    say(f"large-E full size: combine and {toks.size} tokens end to end ({len(used_e)} experts)")
    ros = rr.reshape(c.T, c.k)[toks]
    used = np.unique(ros[ros >= 0])
    rows_f32 = np.zeros((c.M_cap, c.H), np.float32)    # only the rows these tokens read
    rows_f32[used] = F.bf16_to_f32(dn[used])
    want = M.combine(rows_f32, ros.ravel(), wts[toks], 1.0)
    assert np.array_equal(out[toks], want)
    ref = M.prefill_expert_major(c.x[toks], ids[toks], wts[toks], 0, c.E_local, c.A, c.I,
                                 w.w13, w.s13, w.w2, w.s2, clamp=c.clamp, workers=16)
    ok, mx, mean = end_to_end_ok(out[toks], ref.out)
    say(f"  max |d| / max |ref| = {mx:.3e}, mean |d| / rms(ref) = {mean:.3e}")
    assert ok, (mx, mean)


# ------------------------------------------------- GEMM edge layouts

def _gemm_edge_case(ops, counts, A, K, N, seed):
    """Grouped GEMM on hand-made activations: experts with no rows, exactly one
    full 128-row chunk, a full chunk plus one row, single rows, several chunks;
    K of 1..3 k-steps (items shorter than the transfer ring), N with a partial
    256-column tile. Every live row against the oracle, padding untouched."""
    rng = np.random.default_rng(seed)
    E = len(counts)
    ends, prev = [], 0
    for cnt in counts:
        start = ((prev + A - 1) // A) * A
        ends.append(start + cnt)
        prev = start + cnt
    M_cap = max(((prev + A - 1) // A) * A, A)
    xq = rng.integers(0, 256, size=(M_cap, K), dtype=np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x3C                      # no E4M3 NaN codes
    xsb = rng.integers(120, 131, size=(M_cap, K // 32), dtype=np.uint8)
    xs = np.ascontiguousarray(F.pack_ue8m0_words(xsb).T)  # [K/128, M_cap]
    w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ws = rng.integers(120, 131, size=(E, N, K // 32), dtype=np.uint8)
    wp, sp = ops.moe_pack_mx_weights(dev(w), dev(ws))
    out = torch.full((M_cap, N), BF16_SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ends_d = dev(np.asarray(ends, np.int32))
    assert N % 2 == 0
    ops.moe_grouped_gemm1(dev(xq), dev(xs), ends_d, A, wp, sp, out)
    got = host(out)
    live = np.zeros(M_cap, bool)
    for e, rows in enumerate(_expert_rows(ends, A)):
        if rows.size == 0:
            continue
        live[rows] = True
        ab = xsb[rows]
        _, exact, tsum = M.mx_gemm(xq[rows], ab, w[e], ws[e])
        bm = M.block_max_bound(xq[rows], ab, w[e], ws[e])
        ok, _, _ = gemm_within_bound(got[rows], exact, tsum, K, bm)
        assert ok.all(), f"expert {e}: {np.count_nonzero(~ok)} of {ok.size} outside bound"
    assert np.all(got[~live] == BF16_SENT)


@pytest.mark.parametrize("K,N", [(128, 128), (256, 384), (384, 640), (512, 256), (768, 384),
                                 (1152, 256)])
def test_gemm_edge_layouts(ops, K, N):
    """Edge layouts at k-step counts 1-9: the item walker changes item only in
    an item's last 4 steps, so 4 steps (K = 512) have no step without it, 6
    (K = 768) one pipelined pair, 5 and 9 an odd pipelined step."""
    say(f"gemm edge layouts K={K} N={N}")
    _gemm_edge_case(ops, [0, 128, 129, 1, 300, 0, 17], 128, K, N, seed=K + N)


@pytest.mark.parametrize("E,K,N,seed", [(40, 128, 768, 1), (37, 256, 128, 2), (1024, 128, 256, 3)])
def test_gemm_schedule_random_layouts(ops, E, K, N, seed):
    """The cost-ranked schedule on random layouts: partial chunks of every
    size 1-8 row blocks, experts of several full chunks, chunk counts that
    are not a multiple of the 8 XCDs, an odd number of n-tiles (N = 768), a
    partial n-tile (N = 128), more items than blocks, and 1,024 experts (the
    largest rank count and partial-chunk search)."""
    say(f"gemm schedule random layouts E={E} K={K} N={N}")
    rng = np.random.default_rng(100 + seed)
    if E >= 512:
        counts = rng.integers(0, 24, size=E)
    else:
        kind = rng.integers(0, 4, size=E)
        counts = np.where(kind == 0, 0, np.where(kind == 1, rng.integers(1, 129, size=E),
                          np.where(kind == 2, 128 * rng.integers(1, 4, size=E),
                                   rng.integers(129, 520, size=E))))
    _gemm_edge_case(ops, [int(c) for c in counts], 128, K, N, seed=seed)


def test_gemm_all_empty_writes_nothing(ops):
    say("gemm all-empty")
    _gemm_edge_case(ops, [0, 0, 0], 128, 256, 256, seed=5)


# ------------------------------------------------- fused GEMM1 + act-quant

def _fused_vs_two_call(ops, xq, xs, ends, A, w13, s13, clamp):
    """(hq, hs) of moe_grouped_gemm1_act_quant and of moe_grouped_gemm1 ->
    moe_act_quant_liverows, both on sentinel-filled buffers."""
    M_cap = xq.shape[0]
    E, twoI, _ = w13.shape
    I = twoI // 2
    ends_d = dev(np.asarray(ends, np.int32))
    wp, sp = ops.moe_pack_mx_weights(dev(w13), dev(s13))
    gp, gs = ops.moe_pack_mx_weights_gateup(dev(w13), dev(s13))
    gateup = torch.full((M_cap, twoI), BF16_SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    outs = []
    for fused in (False, True):
        hq = torch.full((M_cap, I), BYTE_SENT, dtype=torch.uint8, device="cuda")
        hs = torch.full((I // 128, M_cap), int(WORD_SENT), dtype=torch.int32, device="cuda")
        if fused:
            ops.moe_grouped_gemm1_act_quant(dev(xq), dev(xs), ends_d, A, gp, gs, clamp, hq, hs)
        else:
            ops.moe_grouped_gemm1(dev(xq), dev(xs), ends_d, A, wp, sp, gateup)
            ops.moe_act_quant_liverows(gateup, ends_d, A, clamp, hq, hs)
        outs.append((host(hq), host(hs)))
    return outs + [host(gateup)]


@pytest.mark.parametrize("I,clamp,H", [(128, 0.0, 256), (256, 6.0, 640), (384, 0.0, 768)])
def test_gemm1_act_quant_fused_equals_two_calls(ops, I, clamp, H):
    """Byte-identical hq / hs against the two-call path on the edge layouts
    (empty, exactly 128, 129, single-row and multi-chunk experts), padding
    untouched; and the two-call path itself against the oracle's act-quant.
    H = 640 and 768 put an odd and an even number of pipelined k-steps
    before the item walker's last 4."""
    say(f"fused gemm1+act-quant I={I} clamp={clamp} H={H}")
    rng = np.random.default_rng(I)
    A = 128
    counts = [0, 128, 129, 1, 300, 0, 17]
    ends, prev = [], 0
    for cnt in counts:
        start = ((prev + A - 1) // A) * A
        ends.append(start + cnt)
        prev = start + cnt
    M_cap = ((prev + A - 1) // A) * A
    xq = rng.integers(0, 256, size=(M_cap, H), dtype=np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x3C
    xsb = rng.integers(118, 128, size=(M_cap, H // 32), dtype=np.uint8)
    xs = np.ascontiguousarray(F.pack_ue8m0_words(xsb).T)
    w13 = rng.integers(0, 256, size=(len(counts), 2 * I, H // 2), dtype=np.uint8)
    s13 = rng.integers(118, 128, size=(len(counts), 2 * I, H // 32), dtype=np.uint8)
    (hq0, hs0), (hq1, hs1), gu = _fused_vs_two_call(ops, xq, xs, ends, A, w13, s13, clamp)
    assert np.array_equal(hq0, hq1) and np.array_equal(hs0, hs1)
    live = np.zeros(M_cap, bool)
    for rows in _expert_rows(ends, A):
        live[rows] = True
    assert np.all(hq1[~live] == BYTE_SENT) and np.all(hs1[:, ~live] == WORD_SENT)
    # the two-call path's act-quant against the oracle's, on the GPU's gateup
    rows = np.flatnonzero(live)
    q, b = M.act_quant_rows(gu[rows], I, clamp)
    assert np.array_equal(hq0[rows], q) and np.array_equal(hs0[:, rows].T, F.pack_ue8m0_words(b))


def test_prefill_fused_chain_equals_unfused_full_size(ops):
    """The prefill EP-share layer through moe_ffn_prefill_fused equals
    moe_ffn_prefill byte for byte (down rows and combined output)."""
    c = W.prefill()
    w = c.weights
    ids, wts = M.route_softmax(c.logits, c.k)
    say("prefill fused chain vs unfused, full size")
    outs = []
    for fused in (False, True):
        buf = ops.alloc_grouped(c.T, c.k, c.E_local, c.M_cap, c.H, c.I, fill=True)
        w13p = (ops.moe_pack_mx_weights_gateup if fused else ops.moe_pack_mx_weights)(dev(w.w13), dev(w.s13))
        w2p = ops.moe_pack_mx_weights(dev(w.w2), dev(w.s2))
        fn = ops.moe_ffn_prefill_fused if fused else ops.moe_ffn_prefill
        y = fn(dev_bf16(c.x), dev(ids), dev(wts), 0, c.A, *w13p, *w2p, buf)
        outs.append((host(buf.hq), host(buf.hs), host(buf.down), host(y)))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_pack_mx_weights_gateup_permutation(ops):
    """moe_pack_mx_weights_gateup equals moe_pack_mx_weights of w13 with its
    16-row blocks reordered as documented (gate / up pairs per 128 columns)."""
    rng = np.random.default_rng(77)
    for E, I, H in ((2, 128, 256), (1, 384, 512)):
        say(f"pack gateup E={E} I={I} H={H}")
        w = rng.integers(0, 256, size=(E, 2 * I, H // 2), dtype=np.uint8)
        s = rng.integers(0, 256, size=(E, 2 * I, H // 32), dtype=np.uint8)
        src = []
        for p in range(2 * I // 16):
            t, l = divmod(p, 16)
            c, k = divmod(l, 4)
            src.append((8 * t + 2 * c + k) if k < 2 else (I // 16 + 8 * t + 2 * c + k - 2))
        rows = (16 * np.asarray(src)[:, None] + np.arange(16)[None, :]).reshape(-1)
        assert sorted(rows.tolist()) == list(range(2 * I))
        gp, gs = ops.moe_pack_mx_weights_gateup(dev(w), dev(s))
        rp, rs = ops.moe_pack_mx_weights(dev(np.ascontiguousarray(w[:, rows])),
                                         dev(np.ascontiguousarray(s[:, rows])))
        assert np.array_equal(host(gp), host(rp)) and np.array_equal(host(gs), host(rs))
