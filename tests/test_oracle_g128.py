"""Pins for the group-128 activation recipe of oracle/moe.py: it agrees with
the pinned group-32 quantiser wherever the two must coincide, its scale
bytes are the smallest UE8M0 powers that cover each 128-column group, its
word packing follows the four-groups-per-word layout, and a contraction with
its scales equals a term-by-term fp64 sum that indexes the scale by k // 128
directly."""
import numpy as np

from oracle import formats as F
from oracle import moe as M


def _bf16_bits(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_g128_equals_g32_when_subgroups_share_amax():
    """A row whose four 32-column blocks of each 128-group hold the same
    largest magnitude quantises identically under both recipes."""
    rng = np.random.default_rng(7)
    R, K = 6, 512
    v = rng.uniform(-0.9, 0.9, size=(R, K)).astype(np.float32)
    peaks = rng.uniform(1.0, 40.0, size=(R, K // 128)).astype(np.float32)
    for r in range(R):
        for g in range(K // 128):
            for s in range(4):
                col = 128 * g + 32 * s + int(rng.integers(0, 32))
                v[r, col] = peaks[r, g] * (1 if s % 2 else -1)
    bits = _bf16_bits(v)
    c32, b32 = M.quant_rows(bits)
    c128, b128 = M.quant_rows_g128(bits)
    assert np.array_equal(c32, c128)
    assert np.array_equal(b32.reshape(R, K // 128, 4), np.repeat(b128[:, :, None], 4, axis=2))


def test_g128_scale_is_the_smallest_covering_power():
    """Per 128-column group: 448 * 2^(b-127) >= amax > 448 * 2^(b-128), and
    every code is within half an e4m3 step of v / 2^(b-127). A group of the
    wrong width breaks one of the two for some group of these rows."""
    rng = np.random.default_rng(11)
    R, K = 8, 1024
    mag = np.exp2(rng.uniform(-12, 12, size=(R, K))).astype(np.float32)
    v = (mag * np.where(rng.random((R, K)) < 0.5, -1, 1)).astype(np.float32)
    bits = _bf16_bits(v)
    vf = F.bf16_to_f32(bits).astype(np.float64)
    codes, b = M.quant_rows_g128(bits)
    assert b.shape == (R, K // 128)
    amax = np.abs(vf).reshape(R, K // 128, 128).max(axis=2)
    sf = np.exp2(b.astype(np.float64) - 127)
    assert np.all(448.0 * sf >= amax)
    assert np.all(448.0 * sf / 2 < amax)
    scaled = vf / np.repeat(sf, 128, axis=1)
    dq = F.e4m3_decode(codes).astype(np.float64)
    step = np.where(np.abs(scaled) >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(np.abs(scaled), 2.0 ** -6))) - 3),
                    2.0 ** -9)
    assert np.all(np.abs(dq - scaled) <= step / 2)


def test_pack_g128_words_layout():
    """Byte j of word c is group 4c + j; bytes past the last group are 0."""
    b = np.arange(1, 11, dtype=np.uint8).reshape(2, 5)
    w = M.pack_g128_words(b).view(np.uint32)
    assert w.tolist() == [[0x04030201, 0x05], [0x09080706, 0x0A]]
    assert M.pack_g128_words(np.zeros((1, 8), np.uint8)).shape == (1, 2)


def test_mx_gemm_with_g128_scales_equals_termwise_sum():
    """mx_gemm with the group-128 bytes expanded to its 32-column blocks
    equals sum_k a_k 2^(b[k//128]-127) w_k 2^(wb[k//32]-127), evaluated term
    by term in fp64 (exact here: scales within a narrow range)."""
    rng = np.random.default_rng(3)
    R, K, N = 3, 256, 5
    aq = rng.integers(0, 256, size=(R, K), dtype=np.uint8)
    aq[(aq & 0x7F) == 0x7F] = 0x38
    b128 = rng.integers(122, 131, size=(R, K // 128), dtype=np.uint8)
    w = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    wb = rng.integers(122, 131, size=(N, K // 32), dtype=np.uint8)
    _, exact, _ = M.mx_gemm(aq, M.expand_g128_bytes(b128), w, wb)
    a = F.e4m3_decode(aq).astype(np.float64)
    wc = F.e2m1_decode(F.e2m1_unpack(w)).astype(np.float64)
    want = np.zeros((R, N))
    for r in range(R):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += (a[r, k] * 2.0 ** (int(b128[r, k // 128]) - 127)
                        * wc[n, k] * 2.0 ** (int(wb[n, k // 32]) - 127))
            want[r, n] = acc
    assert np.array_equal(np.asarray(exact, np.float64), want)
