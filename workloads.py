"""Seeded synthetic inputs for the routed MoE expert FFN.

This module only draws inputs. It holds none of the method's arithmetic
(no routing, no endpoints, no quantisation of activations, no GEMM): both
the CPU oracle and the HIP path consume the arrays it returns, so neither
side can influence what the other is given.

Every generator uses ``numpy.random.Generator(PCG64(seed))`` and draws in
the order written below, so a seed reproduces the same bytes on any
machine. bf16 values are fp32 draws rounded to nearest-even by torch's CPU
cast (a library routine, not code of this project).

The shapes follow the workloads that the source pages measure:

* ``tiny``      - a small layer the oracle finishes in well under a second.
* ``actquant``  - the standalone live-row SiLU*up + FP8 quant benchmark of
  the vLLM live-row review (3,072 live of 28,672 allocated rows, SiLU
  output width 2,048, i.e. gate/up input width 4,096, 32 local experts),
  plus its full-buffer control (all 28,672 rows live).
* ``prefill``   - one GPU's share of an EP8 DeepSeek-V4-style layer at 512
  tokens per GPU: top-6 of 256 experts, 32 local experts, H=4,096,
  I=2,048, Zipf(1.1)-skewed expert loads with two empty local experts.
* ``decode``    - gpt-oss-20b-shaped sparse decode: T in {1,2,4,8},
  32 experts, top-4, H=2,880, gate_up 2,880->5,760, down 2,880->2,880,
  FP8 e4m3 weights with a per-expert fp32 scale (and an MXFP4 variant).
* ``large``     - Kimi-K3-shaped layer: 2,048 tokens, 896 experts, top-16
  sigmoid routing with a selection-only correction bias, latent 3,584,
  intermediate 3,072, clamp 25.0.

The real model inputs the pages used (DeepSeek-V4-Flash layer-10
activations, gpt-oss-20b and Kimi-K3 checkpoints) are not available; these
draws stand in for them with the same shapes, sizes and load skew.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

SEEDS = {"tiny": 1001, "actquant": 1002, "prefill": 1003, "decode": 1004, "large": 1005}

BF16_NAN_SENTINEL = np.uint16(0x7FC1)   # quiet NaN pattern planted in bf16 padding
BYTE_SENTINEL = np.uint8(0xA5)          # planted in u8 / e4m3 padding
WORD_SENTINEL = np.int32(np.uint32(0xA5A5A5A5).view(np.int32))  # packed-scale padding


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even, via torch."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def random_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def mx_scale_bytes(rng: np.random.Generator, shape, lo: int = 123, hi: int = 127) -> np.ndarray:
    """E8M0 scale bytes uniform on [lo, hi], i.e. 2^(lo-127) .. 2^(hi-127)."""
    return rng.integers(lo, hi + 1, size=shape, dtype=np.uint8)


def capacity(T: int, k: int, E_local: int, A: int) -> int:
    """Rows reserved for the grouped layout: every route plus one alignment
    block per local expert, rounded up to a multiple of A (and of 4, the row
    padding of the packed scale layout)."""
    m = T * k + E_local * A
    step = int(np.lcm(A, 4))
    return ((m + step - 1) // step) * step


def zipf_probs(n: int, s: float = 1.1) -> np.ndarray:
    r = np.arange(1, n + 1, dtype=np.float64)
    p = r ** (-s)
    return p / p.sum()


@dataclass
class MxWeights:
    """Packed MXFP4 expert weights: two E2M1 codes per byte (low nibble =
    even column), one E8M0 byte per 32 columns."""
    w13: np.ndarray        # u8 [E, 2I, H/2]   rows 0..I-1 gate, I..2I-1 up
    s13: np.ndarray        # u8 [E, 2I, H/32]
    w2: np.ndarray         # u8 [E, H, I/2]
    s2: np.ndarray         # u8 [E, H, I/32]


@dataclass
class PrefillCase:
    name: str
    T: int                 # tokens whose routes this GPU serves
    E: int                 # global experts
    k: int
    H: int
    I: int
    A: int
    expert_start: int
    E_local: int
    M_cap: int
    score: str             # "softmax" | "sigmoid_bias"
    clamp: float           # <= 0: none
    x: np.ndarray          # bf16 bits [T, H]
    logits: np.ndarray     # fp32 [T, E]
    bias: Optional[np.ndarray]  # fp32 [E] or None
    weights: MxWeights
    own_tokens: int = 0    # tokens routed on this GPU (the prefill EP share routes 512)
    routed_scale: float = 1.0
    meta: dict = field(default_factory=dict)


def _mx_weights(rng, E, H, I) -> MxWeights:
    w13 = random_bytes(rng, (E, 2 * I, H // 2))
    s13 = mx_scale_bytes(rng, (E, 2 * I, H // 32))
    w2 = random_bytes(rng, (E, H, I // 2))
    s2 = mx_scale_bytes(rng, (E, H, I // 32))
    return MxWeights(w13, s13, w2, s2)


def tiny(seed: int = SEEDS["tiny"], T: int = 64, H: int = 256, I: int = 128, E: int = 8,
         k: int = 2, A: int = 128) -> PrefillCase:
    rng = rng_for(seed)
    x = normal_bf16(rng, (T, H))
    logits = rng.standard_normal((T, E), dtype=np.float32)
    w = _mx_weights(rng, E, H, I)
    return PrefillCase("tiny", T, E, k, H, I, A, 0, E, capacity(T, k, E, A), "softmax", 0.0,
                       x, logits, None, w, own_tokens=T)


def prefill_rank_of_expert(e: np.ndarray) -> np.ndarray:
    """Popularity rank (1 = most popular) of global expert e in the EP8 group.
    Local expert j (j < 32) gets rank 8j+3, so every rank's 32 experts span
    all popularity octiles."""
    return 8 * (e % 32) + ((e // 32 + 2) % 8) + 1


def prefill(seed: int = SEEDS["prefill"], tokens_per_gpu: int = 512, ep: int = 8, E: int = 256,
            k: int = 6, H: int = 4096, I: int = 2048, A: int = 128, E_local: int = 32,
            empty_local=(5, 27), with_weights: bool = True) -> PrefillCase:
    """One GPU's share of an EP8 layer. The 8*512 tokens of the EP group
    route top-6 of 256 experts; this GPU owns experts 0..31 and computes the
    rows routed to them. Logits are log-popularity plus Gumbel(0,1) noise, so
    the top-6 of a token's logits is a Zipf(1.1) draw without replacement."""
    rng = rng_for(seed)
    T = tokens_per_gpu * ep
    x = normal_bf16(rng, (T, H))
    e = np.arange(E)
    p = zipf_probs(E)[prefill_rank_of_expert(e) - 1]
    p[list(empty_local)] = 0.0
    p = p / p.sum()
    gumbel = rng.gumbel(0.0, 1.0, size=(T, E))
    with np.errstate(divide="ignore"):
        logp = np.log(p)
    logits = np.where(p[None, :] > 0, logp[None, :] + gumbel, -1e30).astype(np.float32)
    w = _mx_weights(rng, E_local, H, I) if with_weights else None
    return PrefillCase("prefill", T, E, k, H, I, A, 0, E_local, capacity(T, k, E_local, A),
                       "softmax", 0.0, x, logits, None, w, own_tokens=tokens_per_gpu,
                       meta={"ep": ep, "tokens_per_gpu": tokens_per_gpu})


def large(seed: int = SEEDS["large"], T: int = 2048, E: int = 896, k: int = 16, H: int = 3584,
          I: int = 3072, A: int = 128, clamp: float = 25.0, with_weights: bool = True,
          experts_with_weights: Optional[int] = None) -> PrefillCase:
    """Kimi-K3-shaped layer with all 896 experts resident on one GPU."""
    rng = rng_for(seed)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    bias = rng.uniform(-0.05, 0.05, size=E).astype(np.float32)
    x = normal_bf16(rng, (T, H))
    w = None
    if with_weights:
        n = E if experts_with_weights is None else experts_with_weights
        w = _mx_weights(rng, n, H, I)
    return PrefillCase("large", T, E, k, H, I, A, 0, E, capacity(T, k, E, A), "sigmoid_bias",
                       clamp, x, logits, bias, w, own_tokens=T)


@dataclass
class ActQuantCase:
    name: str
    E_local: int
    I: int                  # SiLU output width; gate/up input width is 2I
    A: int
    M_cap: int
    counts: np.ndarray      # int64 [E_local]
    live: np.ndarray        # bf16 bits [sum(counts), 2I]: expert 0's rows, then expert 1's, ...
    clamp: float = 0.0
    gateup: Optional[np.ndarray] = None   # the padded [M_cap, 2I] buffer, once placed


def actquant_counts(seed: int = SEEDS["actquant"], E_local: int = 32, live: int = 3072,
                    empty=(3, 17)) -> np.ndarray:
    rng = rng_for(seed)
    perm = rng.permutation(E_local)
    p = zipf_probs(E_local)[perm]
    p[list(empty)] = 0.0
    p = p / p.sum()
    return rng.multinomial(live, p).astype(np.int64)


def actquant(seed: int = SEEDS["actquant"], full: bool = False, E_local: int = 32, I: int = 2048,
             A: int = 128, M_cap: int = 28672, live: int = 3072,
             counts: Optional[np.ndarray] = None) -> ActQuantCase:
    """Standalone act-quant input: per-expert live-row counts and the live
    gate/up rows themselves, N(0,1), in expert order. ``full=True`` makes
    every allocated row live (count 896 for each of the 32 experts). Where
    the rows sit in the grouped buffer is the method's business: callers
    place them with ``place_rows`` at the starts of their own layout."""
    if counts is None:
        counts = (np.full(E_local, M_cap // E_local, dtype=np.int64) if full
                  else actquant_counts(seed, E_local, live))
    rng = rng_for(seed + 7919)
    rows = normal_bf16(rng, (int(counts.sum()), 2 * I))
    return ActQuantCase("actquant-full" if full else "actquant", E_local, I, A, M_cap,
                        counts, rows)


def place_rows(live: np.ndarray, counts: np.ndarray, starts: np.ndarray, M_cap: int,
               fill=BF16_NAN_SENTINEL) -> np.ndarray:
    """Copy expert e's block of ``live`` (counts[e] rows, experts in order) to
    rows [starts[e], starts[e] + counts[e]) of an [M_cap, width] buffer whose
    other rows hold ``fill``. Pure data movement: the starts come from the
    caller's layout."""
    out = np.full((M_cap, live.shape[1]), fill, dtype=live.dtype)
    src = 0
    for c, st in zip(np.asarray(counts, np.int64), np.asarray(starts, np.int64)):
        c, st = int(c), int(st)
        if c:
            out[st:st + c] = live[src:src + c]
        src += c
    return out


@dataclass
class DecodeCase:
    name: str
    T: int
    E: int
    k: int
    H: int                  # K of gate_up and of down; N of down
    N_gu: int               # 2 * H
    wfmt: str               # "fp8" | "mxfp4"
    x: np.ndarray           # bf16 bits [T, H]
    logits: np.ndarray      # fp32 [T, E]
    w_gu: np.ndarray        # fp8: u8 [E, N_gu, H]; mxfp4: u8 [E, N_gu, H/2]
    s_gu: np.ndarray        # fp8: f32 [E]; mxfp4: u8 [E, N_gu, H/32]
    b_gu: np.ndarray        # bf16 bits [E, N_gu]
    w_d: np.ndarray
    s_d: np.ndarray
    b_d: np.ndarray
    glu_alpha: float = 1.702
    glu_beta: float = 1.0
    glu_limit: float = 7.0


def _e4m3_normal_table() -> np.ndarray:
    """65,536-entry table of e4m3 codes whose empirical distribution is that
    of N(0,1) * 112 rounded to e4m3 (inverse-CDF sampling); drawing a uniform
    16-bit index and looking it up is a fast way to make FP8 weights with a
    normal shape. Built with torch's e4m3 cast."""
    from scipy.special import ndtri
    u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    # the two extreme tails (|z| > 448) saturate to +-448, the largest finite code
    z = np.clip(ndtri(u) * 112.0, -448.0, 448.0).astype(np.float32)
    return torch.from_numpy(z).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def decode(T: int = 1, seed: int = SEEDS["decode"], wfmt: str = "fp8", E: int = 32, k: int = 4,
           H: int = 2880, experts: Optional[int] = None) -> DecodeCase:
    """gpt-oss-20b-shaped decode MoE. ``experts`` limits how many experts get
    weights (the rest of the routing still spans E); used for small tests."""
    rng = rng_for(seed + 17 * T + (0 if wfmt == "fp8" else 1))
    x = normal_bf16(rng, (T, H))
    logits = rng.standard_normal((T, E), dtype=np.float32)
    n = E if experts is None else experts
    N_gu = 2 * H
    if wfmt == "fp8":
        table = _e4m3_normal_table()
        w_gu = table[rng.integers(0, 65536, size=(n, N_gu, H), dtype=np.uint16)]
        w_d = table[rng.integers(0, 65536, size=(n, H, H), dtype=np.uint16)]
        # weights ~ N(0, 0.02^2): codes are N(0,1)*112, so the scale is 0.02/112
        s_gu = (0.02 / 112.0 * rng.uniform(0.8, 1.2, size=n)).astype(np.float32)
        s_d = (0.02 / 112.0 * rng.uniform(0.8, 1.2, size=n)).astype(np.float32)
    elif wfmt == "mxfp4":
        w_gu = random_bytes(rng, (n, N_gu, H // 2))
        s_gu = mx_scale_bytes(rng, (n, N_gu, H // 32), 119, 123)
        w_d = random_bytes(rng, (n, H, H // 2))
        s_d = mx_scale_bytes(rng, (n, H, H // 32), 119, 123)
    else:
        raise ValueError(wfmt)
    b_gu = to_bf16_bits(0.1 * rng.standard_normal((n, N_gu), dtype=np.float32))
    b_d = to_bf16_bits(0.1 * rng.standard_normal((n, H), dtype=np.float32))
    return DecodeCase(f"decode-{wfmt}-T{T}", T, E, k, H, N_gu, wfmt, x, logits,
                      w_gu, s_gu, b_gu, w_d, s_d, b_d)
