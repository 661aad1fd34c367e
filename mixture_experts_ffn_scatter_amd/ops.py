"""Torch binding of the C ABI in ``include/moe_ffn.h``.

Argument marshalling only: each function checks device, dtype, contiguity
and shape of its tensors, derives the integer sizes from the shapes, and
passes raw device pointers plus the current HIP stream to the library.
Every step of the computation runs in the library's kernels. Outputs are
caller-allocated (so callers can plant sentinels in padding); helpers below
allocate them with the right shapes.

bf16 tensors may be ``torch.bfloat16`` or 16-bit integer views of the same
bits; E4M3 / packed E2M1 / E8M0 tensors are ``torch.uint8``; packed UE8M0
scale words are ``torch.int32``.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from ._lib import check, lib

SCORE_FN = {"softmax": 0, "sigmoid_bias": 1}
WFMT = {"fp8": 0, "mxfp4": 1}
_BF16 = (torch.bfloat16, torch.int16, getattr(torch, "uint16", torch.int16))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _req(t: torch.Tensor, name: str, dtypes, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


# ---------------------------------------------------------------- routing

def moe_route(logits: torch.Tensor, k: int, score_fn: str = "softmax",
              correction_bias: Optional[torch.Tensor] = None,
              topk_ids: Optional[torch.Tensor] = None,
              topk_weights: Optional[torch.Tensor] = None):
    _req(logits, "logits", (torch.float32,))
    T, E = logits.shape
    if correction_bias is not None:
        _req(correction_bias, "correction_bias", (torch.float32,), (E,))
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_weights is None:
        topk_weights = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _req(topk_ids, "topk_ids", (torch.int32,), (T, k))
    _req(topk_weights, "topk_weights", (torch.float32,), (T, k))
    st = lib().moe_route(_ptr(logits), T, E, k, SCORE_FN[score_fn], _ptr(correction_bias),
                         _ptr(topk_ids), _ptr(topk_weights), _stream())
    check(st, "moe_route")
    return topk_ids, topk_weights


# ---------------------------------------------------------------- scatter

def moe_scatter_workspace_bytes(T: int, k: int, E_local: int) -> int:
    return int(lib().moe_scatter_workspace_bytes(T, k, E_local))


@dataclass
class GroupedBuffers:
    expert_ends: torch.Tensor   # int32 [E_local]
    route_row: torch.Tensor     # int32 [T*k]
    xq: torch.Tensor            # u8 [M_cap, H]
    xs: torch.Tensor            # int32 [H/128, M_cap]
    workspace: torch.Tensor     # u8
    gateup: torch.Tensor        # bf16 [M_cap, 2I]
    hq: torch.Tensor            # u8 [M_cap, I]
    hs: torch.Tensor            # int32 [I/128, M_cap]
    down: torch.Tensor          # bf16 [M_cap, H]
    out: torch.Tensor           # bf16 [T, H]


def scale_words(K: int, group: int = 32) -> int:
    """Packed UE8M0 words per row for K columns: K/128 for group 32 (four
    per-32 bytes a word), ceil(K/512) for group 128 (four per-128 bytes)."""
    if group == 32:
        return K // 128
    if group == 128:
        return (K + 511) // 512
    raise ValueError(f"activation group {group} (32 or 128)")


def alloc_grouped(T, k, E_local, M_cap, H, I, device="cuda", fill: bool = False,
                  group: int = 32) -> GroupedBuffers:
    """Allocate every buffer of the prefill chain. ``fill=True`` plants the
    padding sentinels (bf16 NaN 0x7FC1, byte 0xA5, word 0xA5A5A5A5)."""
    def u8(*s):
        t = torch.empty(s, dtype=torch.uint8, device=device)
        if fill:
            t.fill_(0xA5)
        return t

    def i32(*s):
        t = torch.empty(s, dtype=torch.int32, device=device)
        if fill:
            t.fill_(-1515870811)  # 0xA5A5A5A5
        return t

    def bf(*s):
        t = torch.empty(s, dtype=torch.int16, device=device)
        if fill:
            t.fill_(0x7FC1)
        return t.view(torch.bfloat16)

    ws = max(moe_scatter_workspace_bytes(T, k, E_local), 1)
    return GroupedBuffers(
        expert_ends=torch.empty(E_local, dtype=torch.int32, device=device),
        route_row=torch.empty(T * k, dtype=torch.int32, device=device),
        xq=u8(M_cap, H), xs=i32(scale_words(H, group), M_cap),
        workspace=torch.empty(ws, dtype=torch.uint8, device=device),
        gateup=bf(M_cap, 2 * I), hq=u8(M_cap, I), hs=i32(scale_words(I, group), M_cap),
        down=bf(M_cap, H), out=bf(T, H))


def moe_scatter_endpoints(topk_ids, expert_start: int, E_local: int, A: int, x,
                          expert_ends, route_row, xq, xs, workspace, group: int = 32):
    _req(topk_ids, "topk_ids", (torch.int32,))
    T, k = topk_ids.shape
    _req(x, "x", _BF16)
    H = x.shape[1]
    M_cap = xq.shape[0]
    _req(x, "x", _BF16, (T, H))
    _req(expert_ends, "expert_ends", (torch.int32,), (E_local,))
    _req(route_row, "route_row", (torch.int32,), (T * k,))
    _req(xq, "xq", (torch.uint8,), (M_cap, H))
    _req(xs, "xs", (torch.int32,), (scale_words(H, group), M_cap))
    _req(workspace, "workspace", (torch.uint8,))
    fn = lib().moe_scatter_endpoints if group == 32 else lib().moe_scatter_endpoints_g128
    st = fn(_ptr(topk_ids), T, k, expert_start, E_local, A, M_cap,
                                     _ptr(x), H, _ptr(expert_ends), _ptr(route_row), _ptr(xq),
                                     _ptr(xs), _ptr(workspace), workspace.numel(), _stream())
    check(st, "moe_scatter_endpoints" + ("" if group == 32 else "_g128"))


def moe_scatter_endpoints_noalloc(topk_ids, expert_start: int, E_local: int, A: int, x,
                                  expert_ends, route_row, xq, xs):
    """moe_scatter_endpoints (group-32 recipe) with the library's static
    per-GPU scratch in place of a workspace: allocates nothing."""
    _req(topk_ids, "topk_ids", (torch.int32,))
    T, k = topk_ids.shape
    _req(x, "x", _BF16)
    H = x.shape[1]
    M_cap = xq.shape[0]
    _req(x, "x", _BF16, (T, H))
    _req(expert_ends, "expert_ends", (torch.int32,), (E_local,))
    _req(route_row, "route_row", (torch.int32,), (T * k,))
    _req(xq, "xq", (torch.uint8,), (M_cap, H))
    _req(xs, "xs", (torch.int32,), (scale_words(H), M_cap))
    st = lib().moe_scatter_endpoints_noalloc(_ptr(topk_ids), T, k, expert_start, E_local, A, M_cap,
                                             _ptr(x), H, _ptr(expert_ends), _ptr(route_row),
                                             _ptr(xq), _ptr(xs), _stream())
    check(st, "moe_scatter_endpoints_noalloc")


# ------------------------------------------------------------------ GEMMs

def packed_scale_shape(E: int, N: int, K: int):
    return (E, K // 128, N // 64, 64, 4)


def moe_pack_mx_weights(w, w_scale):
    """Load-time weight preparation: MXFP4 codes u8 [E, N, K/2] and E8M0
    scales u8 [E, N, K/32] -> (codes in fragment order, same shape [E, N, K/2];
    scales u8 [E, K/128, N/64, 64, 4]: per k-step and group of 4 column
    blocks, one 4-byte word per MFMA lane), the operands of the grouped GEMMs."""
    _req(w, "w", (torch.uint8,))
    E, N, K2 = w.shape
    K = 2 * K2
    _req(w_scale, "w_scale", (torch.uint8,), (E, N, K // 32))
    wp = torch.empty_like(w)
    sp = torch.empty(packed_scale_shape(E, N, K), dtype=torch.uint8, device=w.device)
    st = lib().moe_pack_mx_weights(_ptr(w), _ptr(w_scale), E, N, K, _ptr(wp), _ptr(sp), _stream())
    check(st, "moe_pack_mx_weights")
    return wp, sp


def moe_pack_mx_weights_gateup(w13, w13_scale):
    """moe_pack_mx_weights for the fused GEMM1 + activation path: w13 u8
    [E, 2I, H/2] and its scales -> the same packed shapes with the column
    blocks of gate and up interleaved per 128-column slice of h."""
    _req(w13, "w13", (torch.uint8,))
    E, twoI, H2 = w13.shape
    H = 2 * H2
    _req(w13_scale, "w13_scale", (torch.uint8,), (E, twoI, H // 32))
    wp = torch.empty_like(w13)
    sp = torch.empty(packed_scale_shape(E, twoI, H), dtype=torch.uint8, device=w13.device)
    st = lib().moe_pack_mx_weights_gateup(_ptr(w13), _ptr(w13_scale), E, twoI // 2, H, _ptr(wp),
                                          _ptr(sp), _stream())
    check(st, "moe_pack_mx_weights_gateup")
    return wp, sp


def moe_grouped_gemm1_act_quant(xq, xs, expert_ends, A: int, w13_gateup_packed,
                                w13_gateup_scale_packed, clamp_limit: float, hq, hs,
                                group: int = 32):
    """``group`` 128: moe_grouped_gemm1_act_quant_g128 (xs and hs hold one
    UE8M0 byte per 128 columns)."""
    M_cap, H = xq.shape
    E_local, twoI, _ = w13_gateup_packed.shape
    I = twoI // 2
    _req(xq, "xq", (torch.uint8,))
    _req(xs, "xs", (torch.int32,), (scale_words(H, group), M_cap))
    _req(expert_ends, "expert_ends", (torch.int32,), (E_local,))
    _req(w13_gateup_packed, "w13_gateup_packed", (torch.uint8,), (E_local, 2 * I, H // 2))
    _req(w13_gateup_scale_packed, "w13_gateup_scale_packed", (torch.uint8,),
         packed_scale_shape(E_local, 2 * I, H))
    _req(hq, "hq", (torch.uint8,), (M_cap, I))
    _req(hs, "hs", (torch.int32,), (scale_words(I, group), M_cap))
    fn = lib().moe_grouped_gemm1_act_quant if group == 32 else lib().moe_grouped_gemm1_act_quant_g128
    st = fn(_ptr(xq), _ptr(xs), _ptr(expert_ends), E_local, A, M_cap, H, I,
            _ptr(w13_gateup_packed), _ptr(w13_gateup_scale_packed), float(clamp_limit), _ptr(hq),
            _ptr(hs), _stream())
    check(st, "moe_grouped_gemm1_act_quant" + ("" if group == 32 else "_g128"))


def moe_grouped_gemm1(xq, xs, expert_ends, A: int, w13_packed, w13_scale_packed, gateup,
                      group: int = 32):
    M_cap, H = xq.shape
    E_local, twoI, _ = w13_packed.shape
    I = twoI // 2
    _req(xq, "xq", (torch.uint8,))
    _req(xs, "xs", (torch.int32,), (scale_words(H, group), M_cap))
    _req(expert_ends, "expert_ends", (torch.int32,), (E_local,))
    _req(w13_packed, "w13_packed", (torch.uint8,), (E_local, 2 * I, H // 2))
    _req(w13_scale_packed, "w13_scale_packed", (torch.uint8,), packed_scale_shape(E_local, 2 * I, H))
    _req(gateup, "gateup", _BF16, (M_cap, 2 * I))
    fn = lib().moe_grouped_gemm1 if group == 32 else lib().moe_grouped_gemm1_g128
    st = fn(_ptr(xq), _ptr(xs), _ptr(expert_ends), E_local, A, M_cap, H, I,
            _ptr(w13_packed), _ptr(w13_scale_packed), _ptr(gateup), _stream())
    check(st, "moe_grouped_gemm1" + ("" if group == 32 else "_g128"))


def moe_act_quant_liverows(gateup, expert_ends, A: int, clamp_limit: float, hq, hs,
                           group: int = 32):
    _req(gateup, "gateup", _BF16)
    M_cap, twoI = gateup.shape
    I = twoI // 2
    E_local = expert_ends.shape[0]
    _req(expert_ends, "expert_ends", (torch.int32,), (E_local,))
    _req(hq, "hq", (torch.uint8,), (M_cap, I))
    _req(hs, "hs", (torch.int32,), (scale_words(I, group), M_cap))
    fn = lib().moe_act_quant_liverows if group == 32 else lib().moe_act_quant_liverows_g128
    st = fn(_ptr(gateup), _ptr(expert_ends), E_local, A, M_cap, I,
            float(clamp_limit), _ptr(hq), _ptr(hs), _stream())
    check(st, "moe_act_quant_liverows" + ("" if group == 32 else "_g128"))


def moe_act_quant_liverows_situ(gateup, expert_ends, A: int, hq, hs, situ_beta: float = 4.0,
                                situ_linear_beta: float = 25.0):
    _req(gateup, "gateup", _BF16)
    M_cap, twoI = gateup.shape
    I = twoI // 2
    E_local = expert_ends.shape[0]
    _req(expert_ends, "expert_ends", (torch.int32,), (E_local,))
    _req(hq, "hq", (torch.uint8,), (M_cap, I))
    _req(hs, "hs", (torch.int32,), (I // 128, M_cap))
    st = lib().moe_act_quant_liverows_situ(_ptr(gateup), _ptr(expert_ends), E_local, A, M_cap, I,
                                           float(situ_beta), float(situ_linear_beta), _ptr(hq),
                                           _ptr(hs), _stream())
    check(st, "moe_act_quant_liverows_situ")


def moe_grouped_gemm2(hq, hs, expert_ends, A: int, w2_packed, w2_scale_packed, down,
                      group: int = 32):
    M_cap, I = hq.shape
    E_local, H, _ = w2_packed.shape
    _req(hq, "hq", (torch.uint8,))
    _req(hs, "hs", (torch.int32,), (scale_words(I, group), M_cap))
    _req(expert_ends, "expert_ends", (torch.int32,), (E_local,))
    _req(w2_packed, "w2_packed", (torch.uint8,), (E_local, H, I // 2))
    _req(w2_scale_packed, "w2_scale_packed", (torch.uint8,), packed_scale_shape(E_local, H, I))
    _req(down, "down", _BF16, (M_cap, H))
    fn = lib().moe_grouped_gemm2 if group == 32 else lib().moe_grouped_gemm2_g128
    st = fn(_ptr(hq), _ptr(hs), _ptr(expert_ends), E_local, A, M_cap, I, H,
            _ptr(w2_packed), _ptr(w2_scale_packed), _ptr(down), _stream())
    check(st, "moe_grouped_gemm2" + ("" if group == 32 else "_g128"))


# ------------------------------------------- GEMMs on the checkpoint layout

def moe_grouped_gemm1_natural(xq, xs, expert_ends, A: int, w13, w13_scale, gateup):
    """moe_grouped_gemm1 with w13 u8 [E, 2I, H/2] and its scales u8
    [E, 2I, H/32] as stored in the checkpoint (no packing)."""
    M_cap, H = xq.shape
    E_local, twoI, _ = w13.shape
    I = twoI // 2
    _req(xq, "xq", (torch.uint8,))
    _req(xs, "xs", (torch.int32,), (H // 128, M_cap))
    _req(expert_ends, "expert_ends", (torch.int32,), (E_local,))
    _req(w13, "w13", (torch.uint8,), (E_local, 2 * I, H // 2))
    _req(w13_scale, "w13_scale", (torch.uint8,), (E_local, 2 * I, H // 32))
    _req(gateup, "gateup", _BF16, (M_cap, 2 * I))
    st = lib().moe_grouped_gemm1_natural(_ptr(xq), _ptr(xs), _ptr(expert_ends), E_local, A, M_cap,
                                         H, I, _ptr(w13), _ptr(w13_scale), _ptr(gateup), _stream())
    check(st, "moe_grouped_gemm1_natural")


def moe_grouped_gemm2_natural(hq, hs, expert_ends, A: int, w2, w2_scale, down):
    """moe_grouped_gemm2 with w2 u8 [E, H, I/2] and its scales u8 [E, H, I/32]."""
    M_cap, I = hq.shape
    E_local, H, _ = w2.shape
    _req(hq, "hq", (torch.uint8,))
    _req(hs, "hs", (torch.int32,), (I // 128, M_cap))
    _req(expert_ends, "expert_ends", (torch.int32,), (E_local,))
    _req(w2, "w2", (torch.uint8,), (E_local, H, I // 2))
    _req(w2_scale, "w2_scale", (torch.uint8,), (E_local, H, I // 32))
    _req(down, "down", _BF16, (M_cap, H))
    st = lib().moe_grouped_gemm2_natural(_ptr(hq), _ptr(hs), _ptr(expert_ends), E_local, A, M_cap,
                                         I, H, _ptr(w2), _ptr(w2_scale), _ptr(down), _stream())
    check(st, "moe_grouped_gemm2_natural")


def moe_grouped_gemm1_act_quant_natural(xq, xs, expert_ends, A: int, w13, w13_scale,
                                        clamp_limit: float, hq, hs):
    """moe_grouped_gemm1_act_quant with the checkpoint-layout w13 and scales."""
    M_cap, H = xq.shape
    E_local, twoI, _ = w13.shape
    I = twoI // 2
    _req(xq, "xq", (torch.uint8,))
    _req(xs, "xs", (torch.int32,), (H // 128, M_cap))
    _req(expert_ends, "expert_ends", (torch.int32,), (E_local,))
    _req(w13, "w13", (torch.uint8,), (E_local, 2 * I, H // 2))
    _req(w13_scale, "w13_scale", (torch.uint8,), (E_local, 2 * I, H // 32))
    _req(hq, "hq", (torch.uint8,), (M_cap, I))
    _req(hs, "hs", (torch.int32,), (I // 128, M_cap))
    st = lib().moe_grouped_gemm1_act_quant_natural(_ptr(xq), _ptr(xs), _ptr(expert_ends), E_local,
                                                   A, M_cap, H, I, _ptr(w13), _ptr(w13_scale),
                                                   float(clamp_limit), _ptr(hq), _ptr(hs),
                                                   _stream())
    check(st, "moe_grouped_gemm1_act_quant_natural")


# ------------------------------------------------- masked (E, m_pad, K) slab

@dataclass
class MaskedBuffers:
    masked_m: torch.Tensor      # int32 [E_local]
    route_row: torch.Tensor     # int32 [T*k]
    xq: torch.Tensor            # u8 [E_local, m_pad, H]
    xs: torch.Tensor            # int32 [E_local, H/128, m_pad]
    workspace: torch.Tensor     # u8
    gateup: torch.Tensor        # bf16 [E_local, m_pad, 2I]
    hq: torch.Tensor            # u8 [E_local, m_pad, I]
    hs: torch.Tensor            # int32 [E_local, I/128, m_pad]
    down: torch.Tensor          # bf16 [E_local, m_pad, H]
    out: torch.Tensor           # bf16 [T, H]


def alloc_masked(T, k, E_local, m_pad, H, I, device="cuda", fill: bool = False) -> MaskedBuffers:
    """Allocate every buffer of the chain on the masked slab layout
    (``fill=True`` plants the same padding sentinels as alloc_grouped)."""
    def u8(*s):
        t = torch.empty(s, dtype=torch.uint8, device=device)
        if fill:
            t.fill_(0xA5)
        return t

    def i32(*s):
        t = torch.empty(s, dtype=torch.int32, device=device)
        if fill:
            t.fill_(-1515870811)  # 0xA5A5A5A5
        return t

    def bf(*s):
        t = torch.empty(s, dtype=torch.int16, device=device)
        if fill:
            t.fill_(0x7FC1)
        return t.view(torch.bfloat16)

    ws = max(moe_scatter_workspace_bytes(T, k, E_local), 1)
    return MaskedBuffers(
        masked_m=torch.empty(E_local, dtype=torch.int32, device=device),
        route_row=torch.empty(T * k, dtype=torch.int32, device=device),
        xq=u8(E_local, m_pad, H), xs=i32(E_local, H // 128, m_pad),
        workspace=torch.empty(ws, dtype=torch.uint8, device=device),
        gateup=bf(E_local, m_pad, 2 * I), hq=u8(E_local, m_pad, I), hs=i32(E_local, I // 128, m_pad),
        down=bf(E_local, m_pad, H), out=bf(T, H))


def moe_scatter_masked(topk_ids, expert_start: int, x, masked_m, route_row, xq, xs, workspace):
    _req(topk_ids, "topk_ids", (torch.int32,))
    T, k = topk_ids.shape
    _req(x, "x", _BF16)
    H = x.shape[1]
    _req(xq, "xq", (torch.uint8,))
    E_local, m_pad, _ = xq.shape
    _req(x, "x", _BF16, (T, H))
    _req(xq, "xq", (torch.uint8,), (E_local, m_pad, H))
    _req(masked_m, "masked_m", (torch.int32,), (E_local,))
    _req(route_row, "route_row", (torch.int32,), (T * k,))
    _req(xs, "xs", (torch.int32,), (E_local, H // 128, m_pad))
    _req(workspace, "workspace", (torch.uint8,))
    st = lib().moe_scatter_masked(_ptr(topk_ids), T, k, expert_start, E_local, m_pad, _ptr(x), H,
                                  _ptr(masked_m), _ptr(route_row), _ptr(xq), _ptr(xs),
                                  _ptr(workspace), workspace.numel(), _stream())
    check(st, "moe_scatter_masked")


def moe_grouped_gemm1_masked(xq, xs, masked_m, w13_packed, w13_scale_packed, gateup):
    _req(xq, "xq", (torch.uint8,))
    E_local, m_pad, H = xq.shape
    _, twoI, _ = w13_packed.shape
    I = twoI // 2
    _req(xs, "xs", (torch.int32,), (E_local, H // 128, m_pad))
    _req(masked_m, "masked_m", (torch.int32,), (E_local,))
    _req(w13_packed, "w13_packed", (torch.uint8,), (E_local, 2 * I, H // 2))
    _req(w13_scale_packed, "w13_scale_packed", (torch.uint8,), packed_scale_shape(E_local, 2 * I, H))
    _req(gateup, "gateup", _BF16, (E_local, m_pad, 2 * I))
    st = lib().moe_grouped_gemm1_masked(_ptr(xq), _ptr(xs), _ptr(masked_m), E_local, m_pad, H, I,
                                        _ptr(w13_packed), _ptr(w13_scale_packed), _ptr(gateup),
                                        _stream())
    check(st, "moe_grouped_gemm1_masked")


def moe_act_quant_masked(gateup, masked_m, clamp_limit: float, hq, hs):
    _req(gateup, "gateup", _BF16)
    E_local, m_pad, twoI = gateup.shape
    I = twoI // 2
    _req(masked_m, "masked_m", (torch.int32,), (E_local,))
    _req(hq, "hq", (torch.uint8,), (E_local, m_pad, I))
    _req(hs, "hs", (torch.int32,), (E_local, I // 128, m_pad))
    st = lib().moe_act_quant_masked(_ptr(gateup), _ptr(masked_m), E_local, m_pad, I,
                                    float(clamp_limit), _ptr(hq), _ptr(hs), _stream())
    check(st, "moe_act_quant_masked")


def moe_grouped_gemm1_act_quant_masked(xq, xs, masked_m, w13_gateup_packed,
                                       w13_gateup_scale_packed, clamp_limit: float, hq, hs):
    _req(xq, "xq", (torch.uint8,))
    E_local, m_pad, H = xq.shape
    _, twoI, _ = w13_gateup_packed.shape
    I = twoI // 2
    _req(xs, "xs", (torch.int32,), (E_local, H // 128, m_pad))
    _req(masked_m, "masked_m", (torch.int32,), (E_local,))
    _req(w13_gateup_packed, "w13_gateup_packed", (torch.uint8,), (E_local, 2 * I, H // 2))
    _req(w13_gateup_scale_packed, "w13_gateup_scale_packed", (torch.uint8,),
         packed_scale_shape(E_local, 2 * I, H))
    _req(hq, "hq", (torch.uint8,), (E_local, m_pad, I))
    _req(hs, "hs", (torch.int32,), (E_local, I // 128, m_pad))
    st = lib().moe_grouped_gemm1_act_quant_masked(_ptr(xq), _ptr(xs), _ptr(masked_m), E_local,
                                                  m_pad, H, I, _ptr(w13_gateup_packed),
                                                  _ptr(w13_gateup_scale_packed),
                                                  float(clamp_limit), _ptr(hq), _ptr(hs),
                                                  _stream())
    check(st, "moe_grouped_gemm1_act_quant_masked")


def moe_grouped_gemm2_masked(hq, hs, masked_m, w2_packed, w2_scale_packed, down):
    _req(hq, "hq", (torch.uint8,))
    E_local, m_pad, I = hq.shape
    _, H, _ = w2_packed.shape
    _req(hs, "hs", (torch.int32,), (E_local, I // 128, m_pad))
    _req(masked_m, "masked_m", (torch.int32,), (E_local,))
    _req(w2_packed, "w2_packed", (torch.uint8,), (E_local, H, I // 2))
    _req(w2_scale_packed, "w2_scale_packed", (torch.uint8,), packed_scale_shape(E_local, H, I))
    _req(down, "down", _BF16, (E_local, m_pad, H))
    st = lib().moe_grouped_gemm2_masked(_ptr(hq), _ptr(hs), _ptr(masked_m), E_local, m_pad, I, H,
                                        _ptr(w2_packed), _ptr(w2_scale_packed), _ptr(down),
                                        _stream())
    check(st, "moe_grouped_gemm2_masked")


# ---------------------------------------------------------------- combine

def moe_combine(rows, row_of_slot, topk_weights, routed_scale: float, out):
    _req(rows, "rows", _BF16)
    n_rows, H = rows.shape
    _req(topk_weights, "topk_weights", (torch.float32,))
    T, k = topk_weights.shape
    _req(row_of_slot, "row_of_slot", (torch.int32,), (T * k,))
    _req(out, "out", _BF16, (T, H))
    st = lib().moe_combine(_ptr(rows), n_rows, _ptr(row_of_slot), _ptr(topk_weights), T, k, H,
                           float(routed_scale), _ptr(out), _stream())
    check(st, "moe_combine")


# ------------------------------------------------------------ decode GEMV

def moe_sparse_gemv(act, act_per_slot: bool, topk_ids, expert_start: int, E_local: int,
                    wfmt: str, w, w_scale, bias, out, slot_row=None, glu: bool = False,
                    glu_alpha: float = 1.702, glu_beta: float = 1.0, glu_limit: float = 7.0,
                    glu_on_load: bool = False):
    """``glu``: the GLU in the epilogue (out [T*k, N/2]). ``glu_on_load``: the
    GLU applied to the activation as it is read (act = the per-slot gate/up
    rows [T*k, 2K] of the first GEMV; out [T*k, N])."""
    _req(topk_ids, "topk_ids", (torch.int32,))
    T, k = topk_ids.shape
    _req(act, "act", _BF16)
    if glu and glu_on_load:
        raise ValueError("glu and glu_on_load are exclusive")
    if glu_on_load:
        if not act_per_slot:
            raise ValueError("glu_on_load takes per-slot gate/up rows")
        K = act.shape[1] // 2
        _req(act, "act", _BF16, (T * k, 2 * K))
    else:
        K = act.shape[1]
        _req(act, "act", _BF16, ((T * k) if act_per_slot else T, K))
    _req(w, "w", (torch.uint8,))
    N = w.shape[1]
    if wfmt == "fp8":
        _req(w, "w", (torch.uint8,), (E_local, N, K))
        _req(w_scale, "w_scale", (torch.float32,), (E_local,))
    else:
        _req(w, "w", (torch.uint8,), (E_local, N, K // 2))
        _req(w_scale, "w_scale", (torch.uint8,), (E_local, N, K // 32))
    if bias is not None:
        _req(bias, "bias", _BF16, (E_local, N))
    _req(out, "out", _BF16, (T * k, N // 2 if glu else N))
    if slot_row is not None:
        _req(slot_row, "slot_row", (torch.int32,), (T * k,))
    mode = 2 if glu_on_load else int(bool(glu))
    st = lib().moe_sparse_gemv(_ptr(act), int(bool(act_per_slot)), _ptr(topk_ids), T, k,
                               expert_start, E_local, N, K, WFMT[wfmt], _ptr(w), _ptr(w_scale),
                               _ptr(bias), mode, float(glu_alpha), float(glu_beta),
                               float(glu_limit), _ptr(out), _ptr(slot_row), _stream())
    check(st, "moe_sparse_gemv")


# ------------------------------------------------------------------ chains

def moe_ffn_prefill(x, topk_ids, topk_weights, expert_start: int, A: int, w13_packed,
                    w13_scale_packed, w2_packed, w2_scale_packed, buf: GroupedBuffers,
                    clamp_limit: float = 0.0, routed_scale: float = 1.0):
    """scatter -> GEMM1 -> live-row act-quant -> GEMM2 -> combine, all on the
    current stream, no host synchronisation. Weights are the outputs of
    moe_pack_mx_weights."""
    E_local = w13_packed.shape[0]
    moe_scatter_endpoints(topk_ids, expert_start, E_local, A, x, buf.expert_ends, buf.route_row,
                          buf.xq, buf.xs, buf.workspace)
    moe_grouped_gemm1(buf.xq, buf.xs, buf.expert_ends, A, w13_packed, w13_scale_packed,
                      buf.gateup)
    moe_act_quant_liverows(buf.gateup, buf.expert_ends, A, clamp_limit, buf.hq, buf.hs)
    moe_grouped_gemm2(buf.hq, buf.hs, buf.expert_ends, A, w2_packed, w2_scale_packed, buf.down)
    moe_combine(buf.down, buf.route_row, topk_weights, routed_scale, buf.out)
    return buf.out


def moe_ffn_prefill_fused(x, topk_ids, topk_weights, expert_start: int, A: int,
                          w13_gateup_packed, w13_gateup_scale_packed, w2_packed, w2_scale_packed,
                          buf: GroupedBuffers, clamp_limit: float = 0.0,
                          routed_scale: float = 1.0):
    """moe_ffn_prefill with GEMM1 and the live-row act-quant in one kernel
    (w13 from moe_pack_mx_weights_gateup); byte-identical results, and the
    bf16 gate/up rows (buf.gateup) are never written."""
    E_local = w13_gateup_packed.shape[0]
    moe_scatter_endpoints(topk_ids, expert_start, E_local, A, x, buf.expert_ends, buf.route_row,
                          buf.xq, buf.xs, buf.workspace)
    moe_grouped_gemm1_act_quant(buf.xq, buf.xs, buf.expert_ends, A, w13_gateup_packed,
                                w13_gateup_scale_packed, clamp_limit, buf.hq, buf.hs)
    moe_grouped_gemm2(buf.hq, buf.hs, buf.expert_ends, A, w2_packed, w2_scale_packed, buf.down)
    moe_combine(buf.down, buf.route_row, topk_weights, routed_scale, buf.out)
    return buf.out


def moe_ffn_prefill_natural(x, topk_ids, topk_weights, expert_start: int, A: int, w13,
                            w13_scale, w2, w2_scale, buf: GroupedBuffers,
                            clamp_limit: float = 0.0, routed_scale: float = 1.0):
    """moe_ffn_prefill_fused on the weights in their checkpoint layout (w13
    u8 [E, 2I, H/2] with rows [gate; up] and scales [E, 2I, H/32]; w2 u8
    [E, H, I/2] and [E, H, I/32]): no load-time packing; byte-identical
    results to the packed fused chain."""
    E_local = w13.shape[0]
    moe_scatter_endpoints(topk_ids, expert_start, E_local, A, x, buf.expert_ends, buf.route_row,
                          buf.xq, buf.xs, buf.workspace)
    moe_grouped_gemm1_act_quant_natural(buf.xq, buf.xs, buf.expert_ends, A, w13, w13_scale,
                                        clamp_limit, buf.hq, buf.hs)
    moe_grouped_gemm2_natural(buf.hq, buf.hs, buf.expert_ends, A, w2, w2_scale, buf.down)
    moe_combine(buf.down, buf.route_row, topk_weights, routed_scale, buf.out)
    return buf.out


def moe_ffn_prefill_masked(x, topk_ids, topk_weights, expert_start: int, w13_packed,
                           w13_scale_packed, w2_packed, w2_scale_packed, buf: MaskedBuffers,
                           clamp_limit: float = 0.0, routed_scale: float = 1.0,
                           fused: bool = False):
    """The chain on the masked slab layout: masked scatter -> GEMM1 ->
    varlen act-quant -> GEMM2 -> combine over the slab's rows. ``fused``:
    GEMM1 and the act-quant in one kernel (w13 from
    moe_pack_mx_weights_gateup)."""
    moe_scatter_masked(topk_ids, expert_start, x, buf.masked_m, buf.route_row, buf.xq, buf.xs,
                       buf.workspace)
    if fused:
        moe_grouped_gemm1_act_quant_masked(buf.xq, buf.xs, buf.masked_m, w13_packed,
                                           w13_scale_packed, clamp_limit, buf.hq, buf.hs)
    else:
        moe_grouped_gemm1_masked(buf.xq, buf.xs, buf.masked_m, w13_packed, w13_scale_packed,
                                 buf.gateup)
        moe_act_quant_masked(buf.gateup, buf.masked_m, clamp_limit, buf.hq, buf.hs)
    moe_grouped_gemm2_masked(buf.hq, buf.hs, buf.masked_m, w2_packed, w2_scale_packed, buf.down)
    E_local, m_pad, H = buf.down.shape
    moe_combine(buf.down.view(E_local * m_pad, H), buf.route_row, topk_weights, routed_scale,
                buf.out)
    return buf.out


@dataclass
class DecodeBuffers:
    act: torch.Tensor       # bf16 [T*k, H]
    down: torch.Tensor      # bf16 [T*k, H]
    slot_row: torch.Tensor  # int32 [T*k]
    out: torch.Tensor       # bf16 [T, H]


def alloc_decode(T, k, H, device="cuda", fill: bool = False) -> DecodeBuffers:
    def bf(*s):
        t = torch.empty(s, dtype=torch.int16, device=device)
        if fill:
            t.fill_(0x7FC1)
        return t.view(torch.bfloat16)
    return DecodeBuffers(bf(T * k, H), bf(T * k, H),
                         torch.empty(T * k, dtype=torch.int32, device=device), bf(T, H))


def moe_ffn_decode(x, topk_ids, topk_weights, expert_start: int, E_local: int, wfmt: str,
                   w_gu, s_gu, b_gu, w_d, s_d, b_d, buf: DecodeBuffers, glu_alpha=1.702,
                   glu_beta=1.0, glu_limit=7.0):
    """sparse GEMV gate_up (+bias, GLU fused) -> sparse GEMV down (+bias) ->
    combine that skips non-local slots."""
    moe_sparse_gemv(x, False, topk_ids, expert_start, E_local, wfmt, w_gu, s_gu, b_gu, buf.act,
                    buf.slot_row, glu=True, glu_alpha=glu_alpha, glu_beta=glu_beta,
                    glu_limit=glu_limit)
    moe_sparse_gemv(buf.act, True, topk_ids, expert_start, E_local, wfmt, w_d, s_d, b_d,
                    buf.down, None, glu=False)
    moe_combine(buf.down, buf.slot_row, topk_weights, 1.0, buf.out)
    return buf.out


# ------------------------------------------------------------ graph capture

def capture_graph(launch) -> "torch.cuda.CUDAGraph":
    """Capture ``launch()`` (a sequence of the calls above on fixed buffers)
    into a HIP graph. Every entry point sizes its grid from host-known
    arguments and never reads device data back, so the captured chain stays
    valid when the routing, and with it every count and endpoint, changes
    between replays; the caller rewrites the input buffers in place and
    calls ``replay()``. One eager run on a side stream precedes the capture."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch()
    return graph
