"""Pins for the routing functions of oracle/moe.py: brute-force full sorts,
the k=E case against scipy's softmax, and sigmoid selection against the
softmax selection when the bias is zero."""
import numpy as np
from scipy.special import expit, softmax

from oracle import moe as M


def _brute_topk(row, k):
    return [i for _, i in sorted(((-float(v), i) for i, v in enumerate(row)))[:k]]


def test_softmax_ids_bruteforce_with_ties():
    rng = np.random.default_rng(8)
    for _ in range(300):
        E = int(rng.integers(1, 12))
        k = int(rng.integers(1, E + 1))
        logits = rng.integers(-3, 4, size=(3, E)).astype(np.float32)   # many exact ties
        ids, w = M.route_softmax(logits, k)
        for t in range(3):
            assert ids[t].tolist() == _brute_topk(logits[t], k)
        assert np.all(np.abs(w.astype(np.float64).sum(-1) - 1.0) <= k * 2.0 ** -23)


def test_softmax_weights_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((50, 8)).astype(np.float32)
    ids, w = M.route_softmax(logits, 8)
    full = softmax(logits.astype(np.float64), axis=-1)
    ref = np.take_along_axis(full, ids, axis=-1)
    assert np.allclose(w, ref, rtol=2 ** -22, atol=0)
    # renormalised top-k equals the full softmax renormalised over the selection
    ids2, w2 = M.route_softmax(logits, 3)
    sel = np.take_along_axis(full, ids2, axis=-1)
    assert np.allclose(w2, sel / sel.sum(-1, keepdims=True), rtol=2 ** -22, atol=0)


def test_sigmoid_zero_bias_selects_like_softmax():
    rng = np.random.default_rng(10)
    logits = rng.standard_normal((200, 64)).astype(np.float32)
    ids_s, _ = M.route_softmax(logits, 6)
    ids_g, w_g = M.route_sigmoid_bias(logits, np.zeros(64, np.float32), 6)
    assert np.array_equal(ids_s, ids_g)
    sig = expit(np.take_along_axis(logits, ids_g, -1).astype(np.float64))
    assert np.allclose(w_g, sig / sig.sum(-1, keepdims=True), rtol=2 ** -21, atol=0)


def test_sigmoid_bias_only_selects():
    logits = np.array([[0.0, 0.1, 0.2, 0.3]], np.float32)
    bias = np.array([1.0, 0.0, 0.0, 0.0], np.float32)     # pushes expert 0 to the top
    ids, w = M.route_sigmoid_bias(logits, bias, 2)
    assert ids.tolist() == [[0, 3]]
    s = expit(np.array([0.0, 0.3]))
    assert np.allclose(w[0], s / s.sum(), rtol=2 ** -21)     # weights ignore the bias


def _brute_sigmoid_bias(logits_row, bias, k):
    """Every k-subset of experts, keyed by fl32(fl32(sigma(l)) + b) with sigma
    from scipy's expit in fp64 (then rounded to fp32): the best subset is the
    one whose sorted (-key, index) list is smallest."""
    import itertools
    s = expit(logits_row.astype(np.float64)).astype(np.float32)
    key = (s + bias).astype(np.float32)
    best = None
    for sub in itertools.combinations(range(len(logits_row)), k):
        order = sorted(sub, key=lambda e: (-float(key[e]), e))
        cand = [(-float(key[e]), e) for e in order]
        if best is None or cand < best[0]:
            best = (cand, order)
    ids = best[1]
    sel = s[ids].astype(np.float64)
    return ids, sel / sel.sum()


def test_sigmoid_bias_bruteforce_nonzero_bias():
    """Selection with a non-zero correction bias ("Kimi-K3 on SM120
    FlashInfer MXFP4", Phase 1 call chain: select on sigma + bias, weigh
    by sigma alone), against every k-subset on small expert counts. Logits
    and biases are drawn from a few values so that exact key ties occur."""
    rng = np.random.default_rng(31)
    for _ in range(150):
        E = int(rng.integers(2, 8))
        k = int(rng.integers(1, E + 1))
        logits = (rng.integers(-4, 5, size=(2, E)) * 0.25).astype(np.float32)
        bias = (rng.integers(-2, 3, size=E) * 0.0625).astype(np.float32)
        ids, w = M.route_sigmoid_bias(logits, bias, k)
        for t in range(2):
            bids, bw = _brute_sigmoid_bias(logits[t], bias, k)
            assert ids[t].tolist() == list(bids)
            assert np.allclose(w[t], bw, rtol=2 ** -21, atol=0)


def test_sigmoid_bias_key_is_an_fp32_sum():
    """The key is fl32(sigma + b): a bias below half an ulp of sigma is lost in
    the fp32 add, which turns a strict fp64 preference into a tie that goes
    to the lower expert index. sigma(0) = 0.5 exactly; 2^-25 is half an ulp
    of 0.5, and the tie rounds to even (0.5)."""
    logits = np.zeros((1, 3), np.float32)
    bias = np.array([0.0, 0.0, 2.0 ** -25], np.float32)
    ids, w = M.route_sigmoid_bias(logits, bias, 1)
    assert ids.tolist() == [[0]]              # an fp64 key would pick expert 2
    bias[2] = 2.0 ** -24                      # a whole ulp survives the add
    ids, _ = M.route_sigmoid_bias(logits, bias, 1)
    assert ids.tolist() == [[2]]
    # a bias can reorder experts whose sigmoids differ, and the weights still
    # come from the sigmoids alone
    logits = np.array([[1.0, 0.5, -0.5]], np.float32)
    bias = np.array([-0.3, 0.0, 0.5], np.float32)
    ids, w = M.route_sigmoid_bias(logits, bias, 2)
    s = expit(np.array([1.0, 0.5, -0.5]))
    key = s + np.array([-0.3, 0.0, 0.5])
    assert ids.tolist() == [list(np.argsort(-key)[:2])] == [[2, 1]]
    assert np.allclose(w[0], s[[2, 1]] / s[[2, 1]].sum(), rtol=2 ** -21)
