"""CPU oracle for the routed MoE expert FFN -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct numpy definitions of every step of the hot
path, written from the source pages (each function cites the passage it
follows). Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path (the
HIP library and its Python binding) never imports, calls or links anything
here, and this package imports nothing from the product.

Page keys used in citations:

* "Blackwell FP4 MoE: live-row boundary" - the review of the vLLM live-row
  change (endpoint recurrence, worked example, act-quant contract).
* "Blackwell DeepGEMM FusedMoE (sglang)" - the SGLang v0.5.21 DeepGEMM
  FusedMoE walkthrough (six stages, UE8M0 packing, combine kernel).
* "Phase 20: Sparse MoE Decode" - the xserv sparse decode design.
* "Kimi-K3 on SM120 FlashInfer MXFP4" - the Kimi-K3 SM120 experiment page
  (sigmoid+bias routing, [gate; up] layout, NaN/E8M0 rules).

Parity status per function is listed in ``oracle/moe.py``'s header.
"""
from . import formats, moe  # noqa: F401
