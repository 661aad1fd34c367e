"""CPU oracle of the routed MoE expert FFN -- TEST INFRASTRUCTURE ONLY.

Each function is the plain definition of one step, written from the source
pages (citations per function). Floating point: exact fp64 wherever the
result is mathematically exact (the MX GEMMs), and a fixed fp32 operation
sequence wherever the contract is bit-exact (activation quantisation,
combine). No blocking, fusion or reordering beyond what each definition
states.

Parity pins (see ``tests/test_oracle_*.py``):

* ``route_softmax`` / ``route_sigmoid_bias`` - brute force over full sorts,
  k=E equals the full softmax, sigmoid with zero bias selects like softmax.
* ``endpoints`` / ``scatter_routes`` - the worked example of "Blackwell FP4
  MoE: live-row boundary" section 2 (golden fixture), the closed form, and
  brute-force coverage over small count vectors.
* ``act_quant_rows`` - torch's e4m3 cast and decimal arithmetic pin the
  format and sigmoid steps; special cases pin the activation.
* ``act_quant_rows_situ`` - the scaled tanh against 120-digit decimal
  evaluation and its closed-form properties over every bf16 input; the
  activation's special cases and an fp64 evaluation of the formula.
* ``mx_gemm`` - an independent pure-Python nibble/byte triple loop, one-hot
  rows and scale doubling.
* ``combine`` - identity and skip cases, slot order and rounding order;
  the token-major chain.
* ``scatter_masked`` / ``scales_slab`` / ``prefill_masked`` - a worked
  example by hand (golden fixture), agreement with the aligned layout's
  rows expert by expert, overflow keeps the earliest routes, and the
  per-expert MN-major word layout against an element loop.
* ``gemv`` / ``glu`` - a dense per-expert evaluation and special cases.
  ``glu`` follows a reading of the pages (the GPT-OSS gated-SiLU form with
  alpha, beta, limit), so its formula itself is parity unpinned beyond the
  special cases listed in the tests.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .formats import (E2M1_VALUES, E4M3_VALUES, bf16_to_f32, e2m1_decode, e2m1_unpack,
                      e4m3_decode, e8m0_decode, pack_ue8m0_words, quant_mx_e4m3, round_to_bf16,
                      scaled_tanh_f32, sigmoid_f32)

GROUP = 32

# ------------------------------------------------------------------ routing

def topk_order(keys: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest keys per row, ordered by (key desc, index
    asc). A stable sort of the negated keys gives exactly that order."""
    keys = np.asarray(keys, dtype=np.float32)
    order = np.argsort(-keys, axis=-1, kind="stable")
    return order[:, :k].astype(np.int32)


def route_softmax(logits: np.ndarray, k: int):
    """Top-k softmax routing ("Blackwell DeepGEMM FusedMoE (sglang)",
    section 1: gate scores -> top-k; "Phase 20: Sparse MoE Decode",
    section 1: router GEMV -> topk_softmax).

    ids: the k largest logits, best first, ties to the lower expert index.
    weights: the softmax restricted to the selected k (which equals the full
    softmax renormalised over them), evaluated in fp64 and rounded to fp32.
    """
    logits = np.asarray(logits, dtype=np.float32)
    ids = topk_order(logits, k)
    sel = np.take_along_axis(logits, ids, axis=-1).astype(np.float64)
    e = np.exp(sel - sel[:, :1])
    w = (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)
    return ids, w


def route_sigmoid_bias(logits: np.ndarray, bias: np.ndarray, k: int):
    """Sigmoid routing with a selection-only correction bias ("Kimi-K3 on
    SM120 FlashInfer MXFP4", Phase 1 call chain: sigmoid scores, the bias
    only picks experts, weights come from the unbiased sigmoid, renormalised).

    s_e   = sigma(l_e), correctly rounded to fp32
    key_e = fl32(s_e + b_e)
    ids   = top-k keys (key desc, index asc)
    w     = s_sel / sum(s_sel)   (fp64, rounded to fp32)
    """
    logits = np.asarray(logits, dtype=np.float32)
    s = sigmoid_f32(logits)
    key = (s + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    ids = topk_order(key, k)
    sel = np.take_along_axis(s, ids, axis=-1).astype(np.float64)
    w = (sel / sel.sum(axis=-1, keepdims=True)).astype(np.float32)
    return ids, w


# ------------------------------------------------------- endpoints, scatter

def align_up(x, A):
    return ((np.asarray(x, dtype=np.int64) + A - 1) // A) * A


def endpoints(counts, A: int):
    """Per-expert live ranges of the aligned grouped layout ("Blackwell FP4
    MoE: live-row boundary", section 2):
        start[0] = 0, start[e] = align_up(end[e-1], A), end[e] = start[e] + count[e].
    The same page states the closed form used by the source: start[e] is the
    sum of the preceding counts, each aligned up to A. Both are computed and
    must agree."""
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.shape[0]
    start = np.zeros(E, dtype=np.int64)
    end = np.zeros(E, dtype=np.int64)
    for e in range(E):
        start[e] = 0 if e == 0 else int(align_up(end[e - 1], A))
        end[e] = start[e] + counts[e]
    closed = np.concatenate([[0], np.cumsum(align_up(counts, A))[:-1]]) if E else start
    assert np.array_equal(start, closed), "endpoint recurrence disagrees with the closed form"
    return start, end


@dataclass
class Scatter:
    counts: np.ndarray      # int64 [E_local]
    start: np.ndarray       # int64 [E_local]
    end: np.ndarray         # int64 [E_local]; the int32 expert_ends handed to consumers
    route_row: np.ndarray   # int32 [T*k]; -1 = route not served by this GPU
    local_routes: np.ndarray  # flattened route indices t*k+s served here, ascending
    local_expert: np.ndarray  # local expert of each of them


def scatter_routes(ids: np.ndarray, expert_start: int, E_local: int, A: int) -> Scatter:
    """Grouped-layout scatter ("Blackwell FP4 MoE: live-row boundary",
    section 2: the scatter writes int32 endpoints in its existing step;
    "Blackwell DeepGEMM FusedMoE (sglang)", Appendix C: row <-> token-slot
    map).

    A route (t, s) is local when e = ids[t,s] - expert_start lies in
    [0, E_local). Its row is start[e] plus the number of earlier local routes
    with the same e, earlier meaning flattened order t*k+s. Non-local routes
    (including negative ids) get -1."""
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    e = ids - expert_start
    local = (e >= 0) & (e < E_local)
    counts = np.bincount(e[local], minlength=E_local).astype(np.int64)
    start, end = endpoints(counts, A)
    route_row = np.full(ids.shape[0], -1, dtype=np.int32)
    nxt = start.copy()
    for r in range(ids.shape[0]):
        if local[r]:
            route_row[r] = nxt[e[r]]
            nxt[e[r]] += 1
    assert np.array_equal(nxt, end)
    lr = np.flatnonzero(local)
    return Scatter(counts, start, end, route_row, lr, e[lr])


def live_row_mask(start, end, M_cap: int) -> np.ndarray:
    m = np.zeros(M_cap, dtype=bool)
    for s, e in zip(start, end):
        m[int(s):int(e)] = True
    return m


# ---------------------------------------------------------- quantisation

def quant_rows(x_bf16_bits: np.ndarray):
    """FP8 e4m3 + UE8M0 per-32 quantisation of bf16 rows (the per-token group
    quantiser of "Blackwell DeepGEMM FusedMoE (sglang)", section 2.2.4,
    with group 32 -- the MXFP8 activation recipe of its quant table)."""
    return quant_mx_e4m3(bf16_to_f32(x_bf16_bits), GROUP)


def act_rows_f32(gateup_bits: np.ndarray, I: int, clamp: float = 0.0) -> np.ndarray:
    """Gated SiLU of gate/up rows, kept in fp32 (the fused act+quant kernels
    of "Blackwell DeepGEMM FusedMoE (sglang)", section 2.4.1:
    silu_mul_keep_fp32, and the clamp of its default branch: up clamped on
    both sides, gate clamped above only). Rows are [gate (I) | up (I)], the
    [gate; up] halves of "Kimi-K3 on SM120 FlashInfer MXFP4".

    g = f32(gate), u = f32(up); if clamp > 0: g = min(g, L), u = min(max(u,-L), L)
    sig = sigma(g) correctly rounded to fp32
    h = fl32(fl32(g * sig) * u)
    """
    gu = bf16_to_f32(gateup_bits)
    g = gu[..., :I].astype(np.float32)
    u = gu[..., I:2 * I].astype(np.float32)
    if clamp > 0:
        L = np.float32(clamp)
        g = np.minimum(g, L)
        u = np.minimum(np.maximum(u, -L), L)
    sig = sigmoid_f32(g)
    s = (g * sig).astype(np.float32)
    return (s * u).astype(np.float32)


def act_quant_rows(gateup_bits: np.ndarray, I: int, clamp: float = 0.0):
    """SiLU*up + FP8/UE8M0 quantisation of live rows ("Blackwell FP4 MoE:
    live-row boundary", sections 1-3: the activation kernel covers only
    [start, end) and leaves padding unwritten)."""
    return quant_mx_e4m3(act_rows_f32(gateup_bits, I, clamp), GROUP)


SITU_BETA_GATE = 4.0     # Kimi-K3's SiTU parameters ("Kimi-K3 on SM120
SITU_BETA_UP = 25.0      # FlashInfer MXFP4": situ_beta 4, situ_linear_beta 25)


def act_rows_f32_situ(gateup_bits: np.ndarray, I: int, beta_g: float = SITU_BETA_GATE,
                      beta_u: float = SITU_BETA_UP) -> np.ndarray:
    """SiTU of gate/up rows, kept in fp32 ("DeepGEMM FusedMoE on Blackwell
    (sglang)", section 2.4.1, situ branch; "Kimi-K3 on SM120 FlashInfer
    MXFP4", the reference formula):

      gate' = beta_g * tanh(g / beta_g) * sigmoid(g),  up' = beta_u * tanh(u / beta_u)
      h = gate' * up'

    taken as the fixed fp32 sequence (every function value correctly rounded
    to fp32, each product rounded once):
      t = fl32(beta_g tanh(g / beta_g)), sig = fl32(sigmoid(g)),
      a = fl32(t * sig), v = fl32(beta_u tanh(u / beta_u)), h = fl32(a * v).
    No clamp: the clamp belongs to the SiLU branch."""
    gu = bf16_to_f32(gateup_bits)
    g = gu[..., :I].astype(np.float32)
    u = gu[..., I:2 * I].astype(np.float32)
    t = scaled_tanh_f32(g, beta_g)
    sig = sigmoid_f32(g)
    a = (t * sig).astype(np.float32)
    v = scaled_tanh_f32(u, beta_u)
    return (a * v).astype(np.float32)


def act_quant_rows_situ(gateup_bits: np.ndarray, I: int, beta_g: float = SITU_BETA_GATE,
                        beta_u: float = SITU_BETA_UP):
    """SiTU + FP8/UE8M0 quantisation of live rows, with the same group-32
    ceil-then-divide quantiser as the SiLU path."""
    return quant_mx_e4m3(act_rows_f32_situ(gateup_bits, I, beta_g, beta_u), GROUP)


def scales_mn_major(bytes_rows: np.ndarray, rows: np.ndarray, M_cap: int, fill=None):
    """Packed UE8M0 words laid out MN-major: word c of row r at [c][r]
    ("Blackwell DeepGEMM FusedMoE (sglang)", section 2.4.1: (K_g/4,
    aligned_m) int32). Rows not listed keep ``fill``."""
    words = pack_ue8m0_words(bytes_rows)           # [R, G/4]
    out = np.full((words.shape[1], M_cap), 0 if fill is None else fill, dtype=np.int32)
    out[:, rows] = words.T
    return out


# ----------------------------------------------- group-128 activation recipe

GROUP_128 = 128


def quant_rows_g128(x_bf16_bits: np.ndarray):
    """The group-128 activation recipe: FP8 e4m3 + UE8M0 per 128 columns
    ("DeepGEMM FusedMoE on Blackwell (sglang)", overview table of quantised
    data types and section 2.1.3: the MXFP4-experts recipe quantises
    activations per (1,128), weights per (1,32)). Same quantiser as
    quant_rows with 128 in place of 32."""
    return quant_mx_e4m3(bf16_to_f32(x_bf16_bits), GROUP_128)


def act_quant_rows_g128(gateup_bits: np.ndarray, I: int, clamp: float = 0.0):
    """act_quant_rows with the group-128 recipe."""
    return quant_mx_e4m3(act_rows_f32(gateup_bits, I, clamp), GROUP_128)


def pack_g128_words(b128: np.ndarray) -> np.ndarray:
    """u8 [R, G] per-128 bytes -> int32 [R, ceil(G/4)]: four consecutive
    groups per word, group 4c+j in byte j of word c ("DeepGEMM FusedMoE on
    Blackwell (sglang)", section 2.2.4: with UE8M0 the scales are int32 words
    of 4 groups, ceil(K/128/4) per token); bytes past the last group are 0."""
    b128 = np.asarray(b128, dtype=np.uint8)
    R, G = b128.shape
    pad = np.zeros((R, (G + 3) // 4 * 4), dtype=np.uint8)
    pad[:, :G] = b128
    return pack_ue8m0_words(pad)


def expand_g128_bytes(b128: np.ndarray) -> np.ndarray:
    """u8 [R, K/128] -> u8 [R, K/32]: a group's scale applies to each of its
    four 32-column blocks (how a per-32 scaled contraction takes it)."""
    return np.repeat(np.asarray(b128, dtype=np.uint8), 4, axis=-1)


# ------------------------------------------------------------------- GEMM

def dequant_e4m3_rows(codes, scale_bytes):
    """code value times 2^(scale - 127) of its 32-column group (fp64, exact)."""
    codes = np.asarray(codes, np.uint8)
    v = e4m3_decode(codes).reshape(codes.shape[:-1] + (-1, GROUP))
    s = e8m0_decode(scale_bytes)[..., None]
    return (v * s).reshape(codes.shape)


# byte -> (value of its low nibble, value of its high nibble): the two E2M1
# elements a byte packs, even column first
_E2M1_BYTE_PAIRS = np.stack([E2M1_VALUES[np.arange(256) & 0xF],
                             E2M1_VALUES[np.arange(256) >> 4]], axis=-1)


def dequant_mxfp4_rows(packed, scale_bytes):
    """E2M1 element value times 2^(scale - 127) of its 32-column group (fp64,
    exact); elements 2i and 2i+1 are the low and high nibble of byte i."""
    packed = np.asarray(packed, np.uint8)
    lead = packed.shape[:-1]
    v = _E2M1_BYTE_PAIRS[packed].reshape(lead + (-1, GROUP))
    s = e8m0_decode(scale_bytes)[..., None]
    return (v * s).reshape(lead + (2 * packed.shape[-1],))


def _code_lsb_table(values: np.ndarray) -> np.ndarray:
    """Exponent of the lowest set bit of each code's value (+large for 0)."""
    out = np.full(values.shape[0], 1 << 20, dtype=np.int64)
    for c, v in enumerate(values):
        if v == 0 or not np.isfinite(v):
            continue
        m, e = np.frexp(abs(v))
        mi = int(np.ldexp(m, 53))
        out[c] = e - 53 + ((mi & -mi).bit_length() - 1)
    return out


_LSB_E4M3 = _code_lsb_table(E4M3_VALUES)
_LSB_E2M1 = _code_lsb_table(E2M1_VALUES)


# per packed E2M1 byte: the smaller lowest-set-bit exponent of its two elements
_LSB_E2M1_BYTE = np.minimum(_LSB_E2M1[np.arange(256) & 0xF], _LSB_E2M1[np.arange(256) >> 4])


def _row_lsb_min(code_lsb: np.ndarray, scale_bytes: np.ndarray, per_group: int = GROUP) -> np.ndarray:
    """Per row: the smallest lowest-set-bit exponent over its non-zero
    entries, where an entry is code * 2^(scale-127) per 32 columns
    (``code_lsb`` holds ``per_group`` values per 32-column group)."""
    s = scale_bytes.astype(np.int64) - 127
    group_min = code_lsb.reshape(code_lsb.shape[0], -1, per_group).min(-1) + s
    return group_min.min(-1)


def block_max_bound(aq, ab, wq_packed, wb, block: int = 128):
    """sum over 128-wide k blocks of max|a| * max|w| in the block, per output:
    an upper bound on the sum over blocks of the largest single product,
    used to bound hardware dot products that align each block's products to
    its largest one."""
    A = np.abs(dequant_e4m3_rows(aq, ab))
    W = np.abs(dequant_mxfp4_rows(wq_packed, wb))
    K = A.shape[1]
    am = A.reshape(A.shape[0], K // block, block).max(-1)
    wm = W.reshape(W.shape[0], K // block, block).max(-1)
    return am @ wm.T


def mx_gemm(aq, ab, wq_packed, wb, check_exact: bool = True):
    """One expert's MX GEMM: out[r, n] = bf16_rne( sum_k a[r,k] * w[n,k] ) with
    a = e4m3(aq) * 2^(ab-127) per 32 columns and w = e2m1(wq) * 2^(wb-127)
    per 32 columns ("Blackwell DeepGEMM FusedMoE (sglang)", sections 2.3 and
    3.3: lhs (M,K) fp8 + scale, rhs (E,N,K//2) packed fp4 + scale,
    out (M,N) bf16).

    The sum is taken in fp64 and is exact: every product is a small integer
    times a power of two, and the check below proves that all partial sums
    are representable. Returns (bf16 bits, exact fp64 sums, sum of |terms|).
    """
    A = dequant_e4m3_rows(aq, ab)
    W = dequant_mxfp4_rows(wq_packed, wb)
    exact = A @ W.T
    tsum = np.abs(A) @ np.abs(W).T
    if check_exact and A.size and W.size:
        # every term is a multiple of 2^(lsb_a + lsb_w); the fp64 sums are exact
        # while the sum of magnitudes stays below 2^53 such units
        la = _row_lsb_min(_LSB_E4M3[np.asarray(aq, np.uint8)], ab)
        lw = _row_lsb_min(_LSB_E2M1_BYTE[np.asarray(wq_packed, np.uint8)], wb, GROUP // 2)
        lsb = la[:, None] + lw[None, :]
        limit = np.ldexp(1.0, np.minimum(lsb + 53, 1000).astype(np.int64))
        bad = (tsum > 0) & (tsum >= limit)
        assert not bad.any(), "fp64 accumulation of the MX GEMM would round"
    return round_to_bf16(exact), exact, tsum


# ---------------------------------------------------------------- combine

def combine(rows_f32: np.ndarray, row_of_slot: np.ndarray, weights: np.ndarray,
            routed_scale: float = 1.0) -> np.ndarray:
    """Weighted top-k combine ("Blackwell DeepGEMM FusedMoE (sglang)",
    section 2.6.1, post_reorder_deepgemm: fp32 sum over the slots whose
    destination row is >= 0, then times routed_scaling_factor; "Phase 20:
    Sparse MoE Decode", section 3: skip non-local slots, never multiply them
    by zero).

    acc = 0.0f; for s = 0..k-1 in order: if row >= 0: acc = fl32(acc + fl32(w*v))
    out = bf16_rne(fl32(acc * routed_scale))
    ``rows_f32`` is indexed by the values of ``row_of_slot``.
    """
    row_of_slot = np.asarray(row_of_slot).reshape(weights.shape)
    T, k = weights.shape
    H = rows_f32.shape[1]
    acc = np.zeros((T, H), dtype=np.float32)
    w = np.asarray(weights, dtype=np.float32)
    for s in range(k):
        r = row_of_slot[:, s]
        m = r >= 0
        if m.any():
            prod = (w[m, s][:, None] * rows_f32[r[m]]).astype(np.float32)
            acc[m] = (acc[m] + prod).astype(np.float32)
    return round_to_bf16((acc * np.float32(routed_scale)).astype(np.float32))


# ------------------------------------------------------------ prefill chain

@dataclass
class PrefillResult:
    scatter: Scatter
    xq: np.ndarray          # u8 [n_local, H]   indexed like scatter.local_routes
    xb: np.ndarray          # u8 [n_local, H/32]
    gateup: np.ndarray      # bf16 [n_local, 2I]
    gateup_exact: np.ndarray
    gateup_tsum: np.ndarray
    hq: np.ndarray          # u8 [n_local, I]
    hb: np.ndarray          # u8 [n_local, I/32]
    down: np.ndarray        # bf16 [n_local, H]
    down_exact: np.ndarray
    down_tsum: np.ndarray
    out: np.ndarray         # bf16 [T, H]


def _expert_major_rows(x_bits, tok, le, E_local, I, w13, s13, w2, s2, clamp, check_exact,
                       workers):
    """The per-row steps of the chain for the placed routes, expert by
    expert: quantise the routed token row, GEMM1, act-quant, GEMM2. ``tok``
    and ``le`` give each placed route's token and local expert, in ascending
    route order (which is ascending row order inside every expert)."""
    n = tok.shape[0]
    H = x_bits.shape[1]
    xq, xb = quant_rows(x_bits[tok]) if n else (np.zeros((0, H), np.uint8),
                                                np.zeros((0, H // GROUP), np.uint8))
    gateup = np.zeros((n, 2 * I), np.uint16)
    gex = np.zeros((n, 2 * I))
    gts = np.zeros((n, 2 * I))
    hq = np.zeros((n, I), np.uint8)
    hb = np.zeros((n, I // GROUP), np.uint8)
    down = np.zeros((n, H), np.uint16)
    dex = np.zeros((n, H))
    dts = np.zeros((n, H))
    def one_expert(e):
        sel = np.flatnonzero(le == e)       # ascending route order == ascending row order
        if sel.size == 0:
            return
        gateup[sel], gex[sel], gts[sel] = mx_gemm(xq[sel], xb[sel], w13[e], s13[e], check_exact)
        hq[sel], hb[sel] = act_quant_rows(gateup[sel], I, clamp)
        down[sel], dex[sel], dts[sel] = mx_gemm(hq[sel], hb[sel], w2[e], s2[e], check_exact)

    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one_expert, np.unique(le)))
    else:
        for e in range(E_local):
            one_expert(e)
    return xq, xb, gateup, gex, gts, hq, hb, down, dex, dts


def prefill_expert_major(x_bits, ids, weights, expert_start, E_local, A, I,
                         w13, s13, w2, s2, clamp=0.0, routed_scale=1.0,
                         check_exact=True, workers: int = 1) -> PrefillResult:
    """The six-step chain in expert-major order ("Blackwell DeepGEMM
    FusedMoE (sglang)", section 1.1 stages 2-6; "Blackwell FP4 MoE: live-row
    boundary", section 2: scatter -> FC1(endpoint) -> SiLU+mul+quant(endpoint)
    -> FC2(endpoint)): scatter, quantise x per route row, GEMM1 per expert,
    act-quant, GEMM2 per expert, combine by route row.

    Experts touch disjoint rows, so ``workers`` > 1 runs the per-expert
    steps on a thread pool; the results are the same arrays."""
    T, k = np.asarray(ids).shape
    H = x_bits.shape[1]
    sc = scatter_routes(ids, expert_start, E_local, A)
    lr, le = sc.local_routes, sc.local_expert
    xq, xb, gateup, gex, gts, hq, hb, down, dex, dts = _expert_major_rows(
        x_bits, lr // k, le, E_local, I, w13, s13, w2, s2, clamp, check_exact, workers)
    # combine reads down rows by their layout row index
    rows = np.zeros((max(int(sc.end.max()) if E_local else 0, 1), H), np.float32)
    rows[sc.route_row[lr]] = bf16_to_f32(down)
    out = combine(rows, sc.route_row, np.asarray(weights, np.float32), routed_scale)
    return PrefillResult(sc, xq, xb, gateup, gex, gts, hq, hb, down, dex, dts, out)


# ------------------------------------------------- masked (E, m_pad, K) slab

@dataclass
class MaskedScatter:
    counts: np.ndarray        # int64 [E_local]: local routes per expert
    masked_m: np.ndarray      # int32 [E_local]: rows present in expert e's slab
    route_row: np.ndarray     # int32 [T*k]: e*m_pad + j, or -1 (not local, or not placed)
    local_routes: np.ndarray  # placed routes t*k+s, ascending
    local_expert: np.ndarray  # local expert of each of them


def scatter_masked(ids: np.ndarray, expert_start: int, E_local: int, m_pad: int) -> MaskedScatter:
    """The masked slab layout ("DeepGEMM FusedMoE on Blackwell (sglang)",
    section 2.2.4, the standard masked pre-permute, and section 3.2, the
    masked grouped GEMM's masked_m): local expert e owns the fixed block of
    m_pad rows [e*m_pad, (e+1)*m_pad) of an [E_local, m_pad, K] buffer. Its
    routes, in flattened route order t*k+s, take rows 0, 1, ... of its block,
    and masked_m[e] is the number of rows taken; the rest of the block is
    padding that no consumer reads.

    The pages size m_pad so that no expert can overflow it (the rank's
    token count rounded up, or the largest masked_m rounded up). Here a
    route whose rank inside its expert reaches m_pad is not placed: its row
    is -1 and masked_m[e] = min(count_e, m_pad)."""
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    e = ids - expert_start
    local = (e >= 0) & (e < E_local)
    counts = np.bincount(e[local], minlength=E_local).astype(np.int64)
    route_row = np.full(ids.shape[0], -1, dtype=np.int32)
    taken = np.zeros(E_local, dtype=np.int64)
    for r in range(ids.shape[0]):
        if local[r] and taken[e[r]] < m_pad:
            route_row[r] = e[r] * m_pad + taken[e[r]]
            taken[e[r]] += 1
    placed = np.flatnonzero(route_row >= 0)
    return MaskedScatter(counts, taken.astype(np.int32), route_row, placed, e[placed])


def scales_slab(bytes_rows: np.ndarray, rows: np.ndarray, E_local: int, m_pad: int, fill=None):
    """Packed UE8M0 words of slab rows, MN-major inside each expert: word c
    of slab row j of expert e at [e][c][j] ("DeepGEMM FusedMoE on Blackwell
    (sglang)", section 3.2: the masked GEMM's activation scales are
    (E, m, G/4) int32 words in MN-major memory; section 2.4.2: the varlen
    act-quant allocates (E, G/4, m) and transposes the view). ``rows`` are
    slab row indices e*m_pad + j; rows not listed keep ``fill``."""
    words = pack_ue8m0_words(bytes_rows)           # [R, G/4]
    out = np.full((E_local, words.shape[1], m_pad), 0 if fill is None else fill, dtype=np.int32)
    e, j = np.divmod(np.asarray(rows, dtype=np.int64), m_pad)
    out[e, :, j] = words
    return out


@dataclass
class MaskedResult:
    scatter: MaskedScatter
    xq: np.ndarray          # u8 [n_placed, H]  indexed like scatter.local_routes
    xb: np.ndarray          # u8 [n_placed, H/32]
    gateup: np.ndarray      # bf16 [n_placed, 2I]
    gateup_exact: np.ndarray
    gateup_tsum: np.ndarray
    hq: np.ndarray          # u8 [n_placed, I]
    hb: np.ndarray          # u8 [n_placed, I/32]
    down: np.ndarray        # bf16 [n_placed, H]
    down_exact: np.ndarray
    down_tsum: np.ndarray
    out: np.ndarray         # bf16 [T, H]


def prefill_masked(x_bits, ids, weights, expert_start, E_local, m_pad, I, w13, s13, w2, s2,
                   clamp=0.0, routed_scale=1.0, check_exact=True,
                   workers: int = 1) -> MaskedResult:
    """The chain on the masked slab layout ("DeepGEMM FusedMoE on Blackwell
    (sglang)": section 2.2.4 masked pre-permute with quantisation, section
    2.3.2 masked GEMM1 over the first masked_m[e] rows of each slab, section
    2.4.2 varlen act-quant bounded by masked_m, section 2.5.2 masked GEMM2,
    then the combine reading each route's row of the (E*m_pad, H) down
    buffer). Per row the steps are those of the aligned layout; only where
    the rows sit differs."""
    T, k = np.asarray(ids).shape
    H = x_bits.shape[1]
    sc = scatter_masked(ids, expert_start, E_local, m_pad)
    lr, le = sc.local_routes, sc.local_expert
    xq, xb, gateup, gex, gts, hq, hb, down, dex, dts = _expert_major_rows(
        x_bits, lr // k, le, E_local, I, w13, s13, w2, s2, clamp, check_exact, workers)
    rows = np.zeros((max(E_local * m_pad, 1), H), np.float32)
    rows[sc.route_row[lr]] = bf16_to_f32(down)
    out = combine(rows, sc.route_row, np.asarray(weights, np.float32), routed_scale)
    return MaskedResult(sc, xq, xb, gateup, gex, gts, hq, hb, down, dex, dts, out)


def prefill_token_major(x_bits, ids, weights, expert_start, E_local, I, w13, s13, w2, s2,
                        clamp=0.0, routed_scale=1.0, tokens=None) -> np.ndarray:
    """Second formulation with no endpoints and no permutation: for each
    token and each slot whose expert is local, quantise the token, run its
    single row through GEMM1, act-quant and GEMM2, and sum the slots in slot
    order ("Blackwell DeepGEMM FusedMoE (sglang)", section 1: every token
    passes its top-k experts and combine sums them by top-k weight).
    Returns bf16 [len(tokens), H]."""
    ids = np.asarray(ids)
    T, k = ids.shape
    H = x_bits.shape[1]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    out = np.zeros((tokens.shape[0], H), np.uint16)
    for i, t in enumerate(tokens):
        xq, xb = quant_rows(x_bits[t:t + 1])
        acc = np.zeros(H, np.float32)
        for s in range(k):
            e = int(ids[t, s]) - expert_start
            if not (0 <= e < E_local):
                continue
            g, _, _ = mx_gemm(xq, xb, w13[e], s13[e])
            hq, hb = act_quant_rows(g, I, clamp)
            d, _, _ = mx_gemm(hq, hb, w2[e], s2[e])
            prod = (np.float32(weights[t, s]) * bf16_to_f32(d[0])).astype(np.float32)
            acc = (acc + prod).astype(np.float32)
        out[i] = round_to_bf16((acc * np.float32(routed_scale)).astype(np.float32))
    return out


# ------------------------------------------------------------- decode GEMV

def gemv_fp8(act_bits, w_codes, w_scale, bias_bits):
    """Rows of activations against one expert's FP8 weights ("Phase 20:
    Sparse MoE Decode", section 3 kernel design: per-output dot product over
    K, epilogue acc * w_scale[expert] + bias[expert, n]).

    acc = fl32(sum_k e4m3(w[n,k]) * f32(act[k]))   (fp64 sum, one rounding)
    y   = bf16_rne(fl32(fl32(acc * s_e) + f32(bias[n])))
    """
    a = bf16_to_f32(act_bits).astype(np.float64)
    W = e4m3_decode(w_codes)
    acc = (a @ W.T).astype(np.float32)
    y = ((acc * np.float32(w_scale)).astype(np.float32)
         + bf16_to_f32(bias_bits)[None, :]).astype(np.float32)
    return round_to_bf16(y), np.abs(a) @ np.abs(W).T * float(w_scale)


def gemv_mxfp4(act_bits, w_packed, w_scale_bytes, bias_bits):
    """MXFP4 variant of ``gemv_fp8``: per-32 E8M0 scales inside the sum and no
    per-expert scale.  y = bf16_rne(fl32(fl32(sum) + f32(bias[n])))."""
    a = bf16_to_f32(act_bits).astype(np.float64)
    W = dequant_mxfp4_rows(w_packed, w_scale_bytes)
    acc = (a @ W.T).astype(np.float32)
    y = (acc + bf16_to_f32(bias_bits)[None, :]).astype(np.float32)
    return round_to_bf16(y), np.abs(a) @ np.abs(W).T


def glu(gate_bits, up_bits, alpha: float, beta: float, limit: float):
    """Gated activation of the decode path, GPT-OSS form ("Kimi-K3 on SM120
    FlashInfer MXFP4", mismatch matrix: SwiGLU alpha=1.702, beta=1,
    limit=7; "Phase 20: Sparse MoE Decode", section 1: bias then GLU):
        g = min(g, limit); u = clamp(u, -limit, limit)
        out = bf16_rne( g * sigma(alpha * g) * (u + beta) )   (fp64, one rounding)
    limit <= 0 disables both clamps."""
    g = bf16_to_f32(gate_bits).astype(np.float64)
    u = bf16_to_f32(up_bits).astype(np.float64)
    if limit > 0:
        g = np.minimum(g, limit)
        u = np.clip(u, -limit, limit)
    with np.errstate(over="ignore"):
        y = g / (1.0 + np.exp(-alpha * g)) * (u + beta)
    return round_to_bf16(y)


@dataclass
class DecodeResult:
    ids: np.ndarray
    weights: np.ndarray
    slot_row: np.ndarray    # int32 [T*k]: t*k+s when local, else -1
    gu: dict                # (t,s) -> bf16 [2H]
    act: dict               # (t,s) -> bf16 [H]
    down: dict              # (t,s) -> bf16 [H]
    out: np.ndarray         # bf16 [T, H]


def decode_chain(case, expert_start: int = 0, E_local: int = None, ids=None, weights=None
                 ) -> DecodeResult:
    """Sparse decode MoE ("Phase 20: Sparse MoE Decode", section 3 data flow:
    router -> sparse GEMV gate_up with bias -> GLU -> sparse GEMV down with
    bias -> weighted sum over local slots only). Computed slot by slot: for
    each (token, slot) whose expert is local, the two GEMVs of that expert."""
    E_local = case.E if E_local is None else E_local
    if ids is None:
        ids, weights = route_softmax(case.logits, case.k)
    T, k = ids.shape
    H = case.H
    slot_row = np.full(T * k, -1, np.int32)
    gu, act, down = {}, {}, {}
    rows = np.zeros((T * k, H), np.float32)
    for t in range(T):
        for s in range(k):
            g = int(ids[t, s])                    # global expert id; the case holds all experts
            if not (0 <= g - expert_start < E_local):
                continue
            e = g
            slot_row[t * k + s] = t * k + s
            if case.wfmt == "fp8":
                g, _ = gemv_fp8(case.x[t:t + 1], case.w_gu[e], case.s_gu[e], case.b_gu[e])
            else:
                g, _ = gemv_mxfp4(case.x[t:t + 1], case.w_gu[e], case.s_gu[e], case.b_gu[e])
            a = glu(g[0, :H], g[0, H:], case.glu_alpha, case.glu_beta, case.glu_limit)
            if case.wfmt == "fp8":
                d, _ = gemv_fp8(a[None, :], case.w_d[e], case.s_d[e], case.b_d[e])
            else:
                d, _ = gemv_mxfp4(a[None, :], case.w_d[e], case.s_d[e], case.b_d[e])
            gu[(t, s)], act[(t, s)], down[(t, s)] = g[0], a, d[0]
            rows[t * k + s] = bf16_to_f32(d[0])
    out = combine(rows, slot_row, weights, 1.0)
    return DecodeResult(ids, weights, slot_row, gu, act, down, out)
