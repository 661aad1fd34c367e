"""The hardware term of the grouped GEMMs' tolerance, measured through the C
ABI on constructed dot products.

The scaled MX matrix instruction of gfx950 (16x16x128, E4M3 activations x
E2M1 weights, one E8M0 scale per 32 elements on each side) does not add its
128 products exactly: it aligns them to the largest and drops low bits. The
GEMM parity tests therefore allow, besides one bf16 rounding on each side
and the fp32 accumulation across 128-wide steps, 2^-10 of the sum over
128-wide blocks of max|a| * max|w|. This test builds single-step dot
products whose exact sums are tiny next to their largest product (a
product and its negation, plus small terms reaching down to about 2^-36 of
it through the group scales) and random wide-range ones, runs them through
moe_grouped_gemm2 with K = 128, and checks that the error beyond the bf16
rounding stays within that term. It prints the largest observed error as
a fraction of the block's largest product."""
import numpy as np
import pytest

from oracle import formats as F
from oracle import moe as M
from tests.gpu_helpers import BF16_SENT, dev, gemm_within_bound, host, say

pytestmark = pytest.mark.gpu

E4M3_448 = 0x7E          # +448, the largest finite E4M3
E2M1_ONE = 0x2           # 1.0


@pytest.fixture(scope="module")
def ops():
    import mixture_experts_ffn_scatter_amd as pkg
    pkg.lib()
    return pkg.ops


def _inputs(seed):
    rng = np.random.default_rng(seed)
    R, K, N = 64, 128, 128
    aq = np.zeros((R, K), np.uint8)
    ab = np.full((R, K // 32), 127, np.uint8)
    for r in range(R):
        if r < 40:
            # +B and -B in group 0 (scale 2^0), small terms elsewhere: group 0
            # holds codes down to the smallest subnormal, groups 1-3 sit about
            # 2^-6, 2^-12, 2^-18 lower (scale bytes near 121, 115, 109)
            k0, k1 = rng.choice(32, size=2, replace=False)
            aq[r] = rng.integers(0x01, 0x30, size=K, dtype=np.uint8) | (
                rng.integers(0, 2, size=K, dtype=np.uint8) << 7)
            aq[r, k0], aq[r, k1] = E4M3_448, E4M3_448 | 0x80
            ab[r] = [127, 121 - (r % 4), 115 - (r % 5), 109 + (r % 3)]
            if r >= 20:                        # no cancellation: a lone large product
                aq[r, k1] = 0
        else:
            # random codes over the whole finite range, scales over 2^-18 .. 2^0
            aq[r] = rng.integers(0, 256, size=K, dtype=np.uint8)
            aq[r][(aq[r] & 0x7F) == 0x7F] = 0x38
            ab[r] = rng.integers(109, 128, size=K // 32, dtype=np.uint8)
    w = np.zeros((1, N, K // 2), np.uint8)
    ws = np.full((1, N, K // 32), 127, np.uint8)
    # columns 0-63: every weight 1.0 (the products are the activations);
    # columns 64-127: random codes and scales 2^-4 .. 2^0
    w[0, :64] = E2M1_ONE | (E2M1_ONE << 4)
    w[0, 64:] = rng.integers(0, 256, size=(64, K // 2), dtype=np.uint8)
    ws[0, 64:] = rng.integers(123, 128, size=(64, K // 32), dtype=np.uint8)
    return aq, ab, w, ws


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_scaled_mfma_error_within_the_block_max_term(ops, seed):
    import torch
    aq, ab, w, ws = _inputs(seed)
    R, K = aq.shape
    N = w.shape[1]
    say(f"scaled MFMA bound seed={seed}: {R} constructed dot products x {N} weight columns")
    hs = np.ascontiguousarray(F.pack_ue8m0_words(ab).T)          # [1, R]
    wp, sp = ops.moe_pack_mx_weights(dev(w), dev(ws))
    down = torch.full((R, N), BF16_SENT, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ends = dev(np.array([R], np.int32))
    ops.moe_grouped_gemm2(dev(aq), dev(hs), ends, 16, wp, sp, down)
    got = host(down)
    _, exact, tsum = M.mx_gemm(aq, ab, w[0], ws[0])
    bm = M.block_max_bound(aq, ab, w[0], ws[0])
    ok, err, _ = gemm_within_bound(got, exact, tsum, K, bm)
    beyond = np.maximum(err - 2.0 ** -8 * np.abs(exact) - 4.0 * 2 * 2.0 ** -24 * tsum, 0.0)
    frac = beyond / np.where(bm > 0, bm, 1.0)
    worst = float(frac.max())
    say(f"  largest error beyond the bf16 rounding: 2^{np.log2(worst):.2f} of the block max product"
        if worst > 0 else "  no error beyond the bf16 rounding")
    assert ok.all(), f"{np.count_nonzero(~ok)} outputs outside the bound"
    # the constructed cancellations do exercise the alignment: some outputs
    # carry an error far above their own bf16 rounding
    assert worst <= 2.0 ** -10
