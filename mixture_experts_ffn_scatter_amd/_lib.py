"""ctypes loader for the in-tree gfx950 library ``libmoe_ffn.so``.

There is no fallback: if the library is missing or its ABI version differs
from the header this binding was written against, loading raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_ffn.so")
ABI_VERSION = 14

c_int, c_i64, c_size, c_float, c_void = (ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                                         ctypes.c_float, ctypes.c_void_p)

# every symbol declared in include/moe_ffn.h, with its argument types
SIGNATURES = {
    "moe_abi_version": (c_int, []),
    "moe_status_string": (ctypes.c_char_p, [c_int]),
    "moe_route": (c_int, [c_void, c_int, c_int, c_int, c_int, c_void, c_void, c_void, c_void]),
    "moe_scatter_workspace_bytes": (c_size, [c_int, c_int, c_int]),
    "moe_scatter_endpoints": (c_int, [c_void, c_int, c_int, c_int, c_int, c_int, c_int, c_void,
                                      c_int, c_void, c_void, c_void, c_void, c_void, c_size,
                                      c_void]),
    "moe_scatter_endpoints_noalloc": (c_int, [c_void, c_int, c_int, c_int, c_int, c_int, c_int,
                                              c_void, c_int, c_void, c_void, c_void, c_void,
                                              c_void]),
    "moe_pack_mx_weights": (c_int, [c_void, c_void, c_int, c_int, c_int, c_void, c_void, c_void]),
    "moe_pack_mx_weights_gateup": (c_int, [c_void, c_void, c_int, c_int, c_int, c_void, c_void, c_void]),
    "moe_grouped_gemm1_act_quant": (c_int, [c_void, c_void, c_void, c_int, c_int, c_int, c_int, c_int,
                                            c_void, c_void, c_float, c_void, c_void, c_void]),
    "moe_grouped_gemm1": (c_int, [c_void, c_void, c_void, c_int, c_int, c_int, c_int, c_int,
                                  c_void, c_void, c_void, c_void]),
    "moe_act_quant_liverows": (c_int, [c_void, c_void, c_int, c_int, c_int, c_int, c_float,
                                       c_void, c_void, c_void]),
    "moe_act_quant_liverows_situ": (c_int, [c_void, c_void, c_int, c_int, c_int, c_int, c_float,
                                            c_float, c_void, c_void, c_void]),
    "moe_grouped_gemm2": (c_int, [c_void, c_void, c_void, c_int, c_int, c_int, c_int, c_int,
                                  c_void, c_void, c_void, c_void]),
    "moe_scatter_endpoints_g128": (c_int, [c_void, c_int, c_int, c_int, c_int, c_int, c_int,
                                           c_void, c_int, c_void, c_void, c_void, c_void, c_void,
                                           c_size, c_void]),
    "moe_grouped_gemm1_g128": (c_int, [c_void, c_void, c_void, c_int, c_int, c_int, c_int, c_int,
                                       c_void, c_void, c_void, c_void]),
    "moe_act_quant_liverows_g128": (c_int, [c_void, c_void, c_int, c_int, c_int, c_int, c_float,
                                            c_void, c_void, c_void]),
    "moe_grouped_gemm2_g128": (c_int, [c_void, c_void, c_void, c_int, c_int, c_int, c_int, c_int,
                                       c_void, c_void, c_void, c_void]),
    "moe_grouped_gemm1_act_quant_g128": (c_int, [c_void, c_void, c_void, c_int, c_int, c_int, c_int,
                                                 c_int, c_void, c_void, c_float, c_void, c_void,
                                                 c_void]),
    "moe_grouped_gemm1_natural": (c_int, [c_void, c_void, c_void, c_int, c_int, c_int, c_int,
                                          c_int, c_void, c_void, c_void, c_void]),
    "moe_grouped_gemm2_natural": (c_int, [c_void, c_void, c_void, c_int, c_int, c_int, c_int,
                                          c_int, c_void, c_void, c_void, c_void]),
    "moe_grouped_gemm1_act_quant_natural": (c_int, [c_void, c_void, c_void, c_int, c_int, c_int,
                                                    c_int, c_int, c_void, c_void, c_float, c_void,
                                                    c_void, c_void]),
    "moe_scatter_masked": (c_int, [c_void, c_int, c_int, c_int, c_int, c_int, c_void, c_int,
                                   c_void, c_void, c_void, c_void, c_void, c_size, c_void]),
    "moe_grouped_gemm1_masked": (c_int, [c_void, c_void, c_void, c_int, c_int, c_int, c_int,
                                         c_void, c_void, c_void, c_void]),
    "moe_act_quant_masked": (c_int, [c_void, c_void, c_int, c_int, c_int, c_float, c_void, c_void,
                                     c_void]),
    "moe_grouped_gemm1_act_quant_masked": (c_int, [c_void, c_void, c_void, c_int, c_int, c_int,
                                                   c_int, c_void, c_void, c_float, c_void, c_void,
                                                   c_void]),
    "moe_grouped_gemm2_masked": (c_int, [c_void, c_void, c_void, c_int, c_int, c_int, c_int,
                                         c_void, c_void, c_void, c_void]),
    "moe_combine": (c_int, [c_void, c_i64, c_void, c_void, c_int, c_int, c_int, c_float, c_void,
                            c_void]),
    "moe_sparse_gemv": (c_int, [c_void, c_int, c_void, c_int, c_int, c_int, c_int, c_int, c_int,
                                c_int, c_void, c_void, c_void, c_int, c_float, c_float, c_float,
                                c_void, c_void, c_void]),
}

_lib = None


class MoeError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mixture_experts_ffn_scatter_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        v = handle.moe_abi_version()
        if v != ABI_VERSION:
            raise MoeError(f"libmoe_ffn.so ABI version {v}, binding expects {ABI_VERSION}")
        _lib = handle
    return _lib


def check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().moe_status_string(status).decode()
        raise MoeError(f"{what} failed with status {status}: {msg}")
