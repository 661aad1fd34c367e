"""MI355X (gfx950) routed MoE expert FFN with a live-row contract.

The compute lives in the HIP library ``libmoe_ffn.so`` (C ABI in
``include/moe_ffn.h``); ``ops`` holds the thin torch binding with the same
entry-point names. PyTorch provides device memory and streams only.
"""
from . import ops  # noqa: F401
from ._lib import ABI_VERSION, LIB_PATH, MoeError, lib  # noqa: F401
