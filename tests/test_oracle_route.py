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
