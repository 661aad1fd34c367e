"""Pins of the oracle's correctly rounded fp32 sigmoid where an fp64
evaluation alone would round the wrong way, and of the stored list of such
inputs (tests/golden/sigmoid_hard_cases.txt).

Closed form: sigma(v) = 1/2 + v/4 - v^3/48 + O(v^5). For v = (2j+1) 2^-23
(0 < v < 2^-14) the linear part lands exactly on the fp32 midpoint
1/2 + (j + 1/2) 2^-24 and the cubic term pulls sigma just below it, so the
correctly rounded value is 1/2 + j 2^-24; for v = -(2j+1) 2^-24 the linear
part lands on 1/2 - (j + 1/2) 2^-25 and the cubic term lifts sigma just
above it, so the value is 1/2 - j 2^-25. fp64 cannot see the cubic term
(it is about 2^-74 at the smallest v) and returns the midpoint itself,
which ties to even: for small j, half of these come out one fp32 step
wrong."""
import os

import numpy as np

from oracle.formats import sigmoid_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sigmoid_hard_cases.txt")


def test_small_positive_inputs_on_a_midpoint_round_down():
    j = np.arange(0, 1024)
    v = ((2 * j + 1) * 2.0 ** -23).astype(np.float32)
    want = (0.5 + j * 2.0 ** -24).astype(np.float32)
    assert np.array_equal(sigmoid_f32(v), want)
    # the plain fp64 evaluation gets the odd-j cases wrong (ties to even)
    naive = (1.0 / (1.0 + np.exp(-v.astype(np.float64)))).astype(np.float32)
    assert np.count_nonzero(naive != want) >= 25


def test_small_negative_inputs_on_a_midpoint_round_up():
    j = np.arange(0, 1024)
    v = (-(2 * j + 1) * 2.0 ** -24).astype(np.float32)
    want = (0.5 - j * 2.0 ** -25).astype(np.float32)
    assert np.array_equal(sigmoid_f32(v), want)
    naive = (1.0 / (1.0 + np.exp(-v.astype(np.float64)))).astype(np.float32)
    assert np.count_nonzero(naive != want) >= 25


def _golden():
    vb, sb = [], []
    with open(GOLDEN) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            a, b = line.split()
            vb.append(int(a, 16))
            sb.append(int(b, 16))
    return (np.array(vb, np.uint32).view(np.float32), np.array(sb, np.uint32).view(np.float32))


def test_hard_case_list_holds_the_closed_form_cases():
    v, s = _golden()
    assert v.size > 1000
    j = np.arange(0, 64)
    for vv, ss in ((((2 * j + 1) * 2.0 ** -23), 0.5 + j * 2.0 ** -24),
                   ((-(2 * j + 1) * 2.0 ** -24), 0.5 - j * 2.0 ** -25)):
        vv, ss = vv.astype(np.float32), ss.astype(np.float32)
        idx = np.searchsorted(np.sort(v.view(np.uint32)), vv.view(np.uint32))
        order = np.argsort(v.view(np.uint32))
        assert np.array_equal(v[order][idx], vv)
        assert np.array_equal(s[order][idx], ss)


def test_hard_case_list_agrees_with_the_oracle_sample():
    v, s = _golden()
    idx = np.linspace(0, v.size - 1, 200).astype(int)
    assert np.array_equal(sigmoid_f32(v[idx]), s[idx])
