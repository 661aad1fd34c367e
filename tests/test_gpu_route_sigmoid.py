"""GPU routing on the inputs where the sigmoid's fp32 rounding is hard to
decide (tests/golden/sigmoid_hard_cases.txt: every fp32 v in (-110, 110)
whose fp64 sigmoid lies within 2^-45 of an fp32 rounding midpoint), through
moe_route with sigmoid + bias scoring.

Each case is one token over three experts: logits [-200, v, -200] and
correction bias [c, 0, c], c = the correctly rounded sigmoid(v). The keys
are then [c, sigmoid(v), c] (sigmoid(-200) rounds to 0), so the top-2 ids
are [0, 1] exactly when the kernel's sigmoid(v) equals c, [1, 0] when it is
above and [0, 2] when it is below: the ids show a one-step error either
way. Expected ids and weights come from the oracle's route_sigmoid_bias."""
import os

import numpy as np
import pytest
import torch

from oracle import moe as M
from tests.gpu_helpers import host, say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sigmoid_hard_cases.txt")


def _cases():
    vb, sb = [], []
    with open(GOLDEN) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            a, b = line.split()
            vb.append(int(a, 16))
            sb.append(int(b, 16))
    return np.array(vb, np.uint32).view(np.float32), np.array(sb, np.uint32).view(np.float32)


def test_route_sigmoid_bias_on_hard_rounding_cases():
    import mixture_experts_ffn_scatter_amd as pkg
    ops = pkg.ops
    v, c = _cases()
    say(f"sigmoid routing on {v.size} hard rounding cases")
    logits = torch.full((1, 3), -200.0, dtype=torch.float32, device="cuda")
    bias = torch.empty(3, dtype=torch.float32, device="cuda")
    ids = torch.empty((1, 2), dtype=torch.int32, device="cuda")
    wts = torch.empty((1, 2), dtype=torch.float32, device="cuda")
    got = np.empty((v.size, 2), np.int32)
    got_w = np.empty((v.size, 2), np.float32)
    for i in range(v.size):
        logits[0, 1] = float(v[i])
        bias.copy_(torch.tensor([c[i], 0.0, c[i]], dtype=torch.float32))
        ops.moe_route(logits, 2, "sigmoid_bias", bias, ids, wts)
        got[i] = host(ids)[0]
        got_w[i] = host(wts)[0]
    want = np.empty_like(got)
    want_w = np.empty_like(got_w)
    for i in range(v.size):
        lg = np.array([[-200.0, v[i], -200.0]], np.float32)
        b = np.array([c[i], 0.0, c[i]], np.float32)
        ii, ww = M.route_sigmoid_bias(lg, b, 2)
        want[i], want_w[i] = ii[0], ww[0]
    assert np.all(want == [0, 1])                 # the construction: a three-way tie
    bad = np.flatnonzero(np.any(got != want, axis=1))
    assert bad.size == 0, [(float(v[i]), got[i].tolist()) for i in bad[:10]]
    assert np.array_equal(got_w, want_w)
