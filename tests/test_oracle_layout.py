"""Pins for the endpoint recurrence and the scatter of oracle/moe.py: the
pages' worked example (golden fixture), invariants that characterise
align_up uniquely, brute force over small count vectors, and a simulated
grid-stride consumer that must cover exactly the live rows."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import moe as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "endpoints_worked_example.json")


def test_worked_example_from_the_page():
    g = json.load(open(GOLDEN))
    start, end = M.endpoints(g["counts"], g["A"])
    assert start.tolist() == g["start"]
    assert end.tolist() == g["end"]


def _check_invariants(counts, A, start, end):
    prev_end = 0
    for e, c in enumerate(counts):
        assert start[e] % A == 0
        assert end[e] - start[e] == c
        # start is the smallest multiple of A that is >= the previous end
        assert start[e] >= prev_end and start[e] - prev_end < A
        prev_end = end[e]


def _simulated_grid_stride(start, end, programs):
    """A consumer launched with `programs` workers per expert that walks
    row = start + i for i = pid, pid+programs, ... while row < end."""
    touched = []
    for e in range(len(start)):
        for pid in range(programs):
            r = start[e] + pid
            while r < end[e]:
                touched.append(int(r))
                r += programs
    return touched


@pytest.mark.parametrize("A", [16, 128])
def test_endpoints_bruteforce_small_vectors(A):
    vals = [0, 1, A - 1, A, A + 1, 2 * A]
    checks = 0
    for E in range(1, 5):
        for counts in itertools.product(vals, repeat=E):
            start, end = M.endpoints(list(counts), A)
            _check_invariants(counts, A, start, end)
            live = M.live_row_mask(start, end, int(M.align_up(end[-1], A)) + A)
            for programs in (1, 3, 64):
                touched = _simulated_grid_stride(start, end, programs)
                assert len(touched) == len(set(touched)) == sum(counts)
                assert np.all(live[touched])
            checks += 1
    assert checks == 6 + 36 + 216 + 1296


def test_endpoints_all_empty_and_full():
    start, end = M.endpoints([0, 0, 0], 128)
    assert start.tolist() == [0, 0, 0] and end.tolist() == [0, 0, 0]
    start, end = M.endpoints([896] * 32, 128)          # every allocated row live
    assert end[-1] == 28672 and np.all(start == np.arange(32) * 896)


def _check_scatter(ids, expert_start, E_local, A):
    sc = M.scatter_routes(ids, expert_start, E_local, A)
    T, k = ids.shape
    flat = ids.reshape(-1)
    # -1 exactly for routes outside the window (negative ids included)
    local = (flat >= expert_start) & (flat < expert_start + E_local)
    assert np.all((sc.route_row >= 0) == local)
    rows = sc.route_row[local]
    assert len(set(rows.tolist())) == rows.size                      # no row twice
    live = M.live_row_mask(sc.start, sc.end, int(sc.end.max(initial=0)) + A)
    assert np.all(live[rows]) and live.sum() == rows.size              # exactly the live rows
    for e in range(E_local):
        routes = np.flatnonzero(flat == expert_start + e)
        assert sc.route_row[routes].tolist() == list(range(sc.start[e], sc.end[e]))  # route order
    _check_invariants(sc.counts, A, sc.start, sc.end)


def test_scatter_bruteforce_random_small():
    rng = np.random.default_rng(7)
    for trial in range(400):
        T = int(rng.integers(0, 12))
        k = int(rng.integers(1, 4))
        E = int(rng.integers(1, 7))
        ids = rng.integers(-1, E + 2, size=(T, k))          # -1 and out-of-window ids
        if trial % 3 == 0 and T:
            ids = np.stack([rng.permutation(E + 2)[:k] - 1 for _ in range(T)]) if k <= E + 2 else ids
        expert_start = int(rng.integers(0, 2))
        A = int(rng.choice([1, 3, 4, 16]))
        _check_scatter(ids.reshape(T, k), expert_start, E, A)


def test_scatter_empty_inputs():
    sc = M.scatter_routes(np.zeros((0, 4), np.int32), 0, 4, 128)
    assert sc.route_row.size == 0 and sc.end.tolist() == [0, 0, 0, 0]
    sc = M.scatter_routes(np.full((5, 2), -1, np.int32), 0, 3, 128)
    assert np.all(sc.route_row == -1) and sc.end.tolist() == [0, 0, 0]
