"""Pins of the oracle's masked (E, m_pad, K) slab layout ("DeepGEMM FusedMoE
on Blackwell (sglang)", sections 2.2.4 and 3.2): a small example worked by
hand from the definition, agreement with the aligned layout (pinned on its
own by the endpoint tests), the overflow rule, the per-expert MN-major word
layout against an element loop, and the chain on the slab against the chain
on the aligned layout."""
import numpy as np
import pytest

import workloads as W
from oracle import moe as M
from oracle.formats import pack_ue8m0_words

# routes r = t*k + s of 4 tokens, top-2: ids 5 and -1 are never local here
IDS = np.array([[2, 0], [0, 1], [2, 5], [-1, 0]], dtype=np.int32)


def test_worked_example_by_hand():
    # expert 0 takes routes 1, 2, 7 (rows 0, 1, 2 of block 0), expert 1
    # route 3 (row 0 of block 1 = 4), expert 2 routes 0, 4 (rows 8, 9)
    sc = M.scatter_masked(IDS, 0, 3, 4)
    assert sc.route_row.tolist() == [8, 0, 1, 4, 9, -1, -1, 2]
    assert sc.masked_m.tolist() == [3, 1, 2]
    assert sc.counts.tolist() == [3, 1, 2]
    assert sc.local_routes.tolist() == [0, 1, 2, 3, 4, 7]
    assert sc.local_expert.tolist() == [2, 0, 0, 1, 2, 0]


def test_worked_example_overflow_by_hand():
    # m_pad 2: expert 0's third route (route 7) finds its block full
    sc = M.scatter_masked(IDS, 0, 3, 2)
    assert sc.route_row.tolist() == [4, 0, 1, 2, 5, -1, -1, -1]
    assert sc.masked_m.tolist() == [2, 1, 2]
    assert sc.counts.tolist() == [3, 1, 2]


def test_worked_example_window_by_hand():
    # experts [1, 3) of the global ids: local expert 0 is id 1, 1 is id 2
    sc = M.scatter_masked(IDS, 1, 2, 4)
    assert sc.route_row.tolist() == [4, -1, -1, 0, 5, -1, -1, -1]
    assert sc.masked_m.tolist() == [1, 2]


def _route_at(route_row, n_rows):
    inv = np.full(n_rows, -1, dtype=np.int64)
    r = np.flatnonzero(route_row >= 0)
    inv[route_row[r]] = r
    return inv


@pytest.mark.parametrize("seed", range(6))
def test_agrees_with_aligned_layout(seed):
    rng = np.random.default_rng(seed)
    T, E = int(rng.integers(1, 80)), int(rng.integers(1, 12))
    k = int(rng.integers(1, min(7, E + 3) + 1))
    ids = np.stack([rng.choice(E + 3, size=k, replace=False) for _ in range(T)]).astype(np.int32) - 1
    es, El = int(rng.integers(0, 2)), int(rng.integers(1, E + 1))
    con = M.scatter_routes(ids, es, El, 16)
    m_pad = int(con.counts.max()) + int(rng.integers(0, 5))
    m_pad = max(m_pad, 1)
    sl = M.scatter_masked(ids, es, El, m_pad)
    assert np.array_equal(sl.counts, con.counts)
    assert np.array_equal(sl.masked_m, con.end - con.start)
    assert np.array_equal(sl.local_routes, con.local_routes)
    a = _route_at(con.route_row, int(con.end.max()) + 1)
    b = _route_at(sl.route_row, El * m_pad)
    for e in range(El):
        n = int(sl.masked_m[e])
        # row j of expert e holds the same route in both layouts
        assert np.array_equal(b[e * m_pad:e * m_pad + n], a[con.start[e]:con.start[e] + n])
        assert np.all(b[e * m_pad + n:(e + 1) * m_pad] == -1)


@pytest.mark.parametrize("seed", range(6))
def test_overflow_keeps_the_earliest_routes(seed):
    rng = np.random.default_rng(100 + seed)
    T, k, E = 60, 4, 6
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    m_pad = int(rng.integers(1, 30))
    sl = M.scatter_masked(ids, 0, E, m_pad)
    flat = ids.reshape(-1)
    for e in range(E):
        routes = np.flatnonzero(flat == e)
        keep, drop = routes[:m_pad], routes[m_pad:]
        assert sl.masked_m[e] == keep.size
        assert sl.route_row[keep].tolist() == [e * m_pad + j for j in range(keep.size)]
        assert np.all(sl.route_row[drop] == -1)


def test_scales_slab_element_loop():
    rng = np.random.default_rng(7)
    E, m_pad, G = 3, 5, 8
    rows = np.array([0, 1, 5, 10, 11, 14])
    b = rng.integers(0, 256, size=(rows.size, G), dtype=np.uint8)
    got = M.scales_slab(b, rows, E, m_pad, fill=-7)
    want = np.full((E, G // 4, m_pad), (-7) % (1 << 32), dtype=np.int64)
    for i, r in enumerate(rows):
        e, j = divmod(int(r), m_pad)
        for c in range(G // 4):
            # group 4c+q in byte q (least significant first)
            want[e, c, j] = sum(int(b[i, 4 * c + q]) << (8 * q) for q in range(4))
    assert np.array_equal(got.view(np.uint32).astype(np.int64), want)
    # the aligned layout's words of the same rows are the same numbers
    assert np.array_equal(pack_ue8m0_words(b), got[rows // m_pad, :, rows % m_pad])


def test_chain_on_slab_equals_chain_on_aligned_layout():
    c = W.tiny()
    w = c.weights
    ids, wts = M.route_softmax(c.logits, c.k)
    con = M.prefill_expert_major(c.x, ids, wts, 0, c.E_local, c.A, c.I, w.w13, w.s13, w.w2, w.s2)
    m_pad = int(con.scatter.counts.max())
    sl = M.prefill_masked(c.x, ids, wts, 0, c.E_local, m_pad, c.I, w.w13, w.s13, w.w2, w.s2)
    assert np.array_equal(sl.out, con.out)
    assert np.array_equal(sl.hq, con.hq) and np.array_equal(sl.down, con.down)


def test_chain_with_overflow_drops_exactly_the_unplaced_routes():
    c = W.tiny()
    w = c.weights
    ids, wts = M.route_softmax(c.logits, c.k)
    m_pad = 12                              # below the busiest experts' counts
    sl = M.prefill_masked(c.x, ids, wts, 0, c.E_local, m_pad, c.I, w.w13, w.s13, w.w2, w.s2)
    assert int(sl.scatter.counts.max()) > m_pad
    dropped = (sl.scatter.route_row < 0).reshape(ids.shape)
    ids_kept = np.where(dropped, -1, ids)
    con = M.prefill_expert_major(c.x, ids_kept, wts, 0, c.E_local, c.A, c.I, w.w13, w.s13, w.w2,
                                 w.s2)
    assert np.array_equal(sl.out, con.out)
