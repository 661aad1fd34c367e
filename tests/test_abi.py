"""CPU-only checks of the C-ABI library: it loads, exports every function
declared in include/*.h with the right ABI version, validates arguments on
the host (these calls return before any GPU work), and the HIP side's
build-time sigmoid table equals the oracle's correctly rounded sigmoid."""
import ctypes
import glob
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "mixture_experts_ffn_scatter_amd", "libmoe_ffn.so")


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", text, re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from mixture_experts_ffn_scatter_amd import build
        build.build(verbose=False)
    from mixture_experts_ffn_scatter_amd import _lib
    return _lib.lib()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"moe_route", "moe_scatter_endpoints", "moe_grouped_gemm1", "moe_act_quant_liverows",
            "moe_grouped_gemm2", "moe_combine", "moe_sparse_gemv"} <= names
    for n in names:
        assert hasattr(lib, n), n
    from mixture_experts_ffn_scatter_amd import _lib
    assert names == set(_lib.SIGNATURES)


def test_abi_version_and_status_strings(lib):
    assert lib.moe_abi_version() == 14
    for s in range(0, -10, -1):
        assert lib.moe_status_string(s).decode()
    assert lib.moe_status_string(5).decode() == "unknown status"


def test_workspace_bytes(lib):
    # per (64-token block, expert) offsets, then one start per expert
    assert lib.moe_scatter_workspace_bytes(4096, 6, 32) == (64 + 1) * 32 * 4
    # blocks double until the block-by-expert table holds <= 32768 counters
    assert lib.moe_scatter_workspace_bytes(65536, 8, 1024) == (32 + 1) * 1024 * 4
    assert lib.moe_scatter_workspace_bytes(2048, 16, 896) == (32 + 1) * 896 * 4
    assert lib.moe_scatter_workspace_bytes(0, 6, 32) == 0


NULL = None


def test_host_validation_returns_errors_without_gpu_work(lib):
    # each call below fails a host-side check before anything is enqueued
    assert lib.moe_route(NULL, 4, 8, 0, 0, NULL, NULL, NULL, NULL) == -2          # k = 0
    assert lib.moe_route(NULL, 4, 8, 9, 0, NULL, NULL, NULL, NULL) == -2          # k > E
    assert lib.moe_route(NULL, 4, 8, 2, 7, NULL, NULL, NULL, NULL) == -5          # bad score fn
    assert lib.moe_route(NULL, 4, 8, 2, 1, NULL, NULL, NULL, NULL) == -1          # bias missing
    assert lib.moe_route(NULL, 0, 8, 2, 0, NULL, NULL, NULL, NULL) == 0           # T = 0: no-op
    # scatter: H not a multiple of 128, capacity too small, workspace too small
    args = [NULL, 64, 2, 0, 8, 128, 1152, NULL, 200, NULL, NULL, NULL, NULL, NULL, 0, NULL]
    assert lib.moe_scatter_endpoints(*args) == -3
    args[8] = 256
    args[6] = 1024
    assert lib.moe_scatter_endpoints(*args) == -4
    args[6] = 1152
    assert lib.moe_scatter_endpoints(*args) == -1                                 # NULL pointers
    # the no-alloc form: the same checks, in the same order, before any
    # device query (there is no workspace argument)
    na = args[:14] + [NULL]
    na[8], na[6] = 200, 1152
    assert lib.moe_scatter_endpoints_noalloc(*na) == -3
    na[8], na[6] = 256, 1024
    assert lib.moe_scatter_endpoints_noalloc(*na) == -4
    na[6] = 1152
    assert lib.moe_scatter_endpoints_noalloc(*na) == -1
    assert lib.moe_scatter_endpoints_noalloc(NULL, 64, 2, 0, 1025, 128, 1 << 20, NULL, 256, NULL,
                                             NULL, NULL, NULL, NULL) == -2        # E_local > 1024
    # act-quant: clamp limit that is not a bf16 value
    assert lib.moe_act_quant_liverows(NULL, NULL, 8, 128, 1152, 128, ctypes.c_float(7.3),
                                      NULL, NULL, NULL) == -5
    assert lib.moe_act_quant_liverows(NULL, NULL, 8, 128, 1152, 100, ctypes.c_float(0.0),
                                      NULL, NULL, NULL) == -3
    # SiTU act-quant: only Kimi-K3's (4, 25); shape checks as for SiLU
    assert lib.moe_act_quant_liverows_situ(NULL, NULL, 8, 128, 1152, 128, ctypes.c_float(4.0),
                                           ctypes.c_float(20.0), NULL, NULL, NULL) == -5
    assert lib.moe_act_quant_liverows_situ(NULL, NULL, 8, 128, 1152, 100, ctypes.c_float(4.0),
                                           ctypes.c_float(25.0), NULL, NULL, NULL) == -3
    assert lib.moe_act_quant_liverows_situ(NULL, NULL, 8, 128, 1152, 128, ctypes.c_float(4.0),
                                           ctypes.c_float(25.0), NULL, NULL, NULL) == -1
    # GEMMs: K not a multiple of 128
    assert lib.moe_grouped_gemm1(NULL, NULL, NULL, 8, 128, 1152, 192, 128, NULL, NULL, NULL,
                                 NULL) == -3
    assert lib.moe_grouped_gemm2(NULL, NULL, NULL, 8, 128, 1152, 100, 256, NULL, NULL, NULL,
                                 NULL) == -3
    # group-128 forms: the same checks as their group-32 counterparts
    args = [NULL, 64, 2, 0, 8, 128, 1152, NULL, 200, NULL, NULL, NULL, NULL, NULL, 0, NULL]
    assert lib.moe_scatter_endpoints_g128(*args) == -3
    args[8] = 256
    assert lib.moe_scatter_endpoints_g128(*args) == -1
    assert lib.moe_act_quant_liverows_g128(NULL, NULL, 8, 128, 1152, 128, ctypes.c_float(7.3),
                                           NULL, NULL, NULL) == -5
    assert lib.moe_act_quant_liverows_g128(NULL, NULL, 8, 128, 1152, 100, ctypes.c_float(0.0),
                                           NULL, NULL, NULL) == -3
    assert lib.moe_grouped_gemm1_g128(NULL, NULL, NULL, 8, 128, 1152, 192, 128, NULL, NULL, NULL,
                                      NULL) == -3
    assert lib.moe_grouped_gemm2_g128(NULL, NULL, NULL, 8, 128, 1152, 100, 256, NULL, NULL, NULL,
                                      NULL) == -3
    assert lib.moe_grouped_gemm2_g128(NULL, NULL, NULL, 8, 128, 1152, 256, 256, NULL, NULL, NULL,
                                      NULL) == -1
    # weight packing: K not a multiple of 128, N not of 64 (the scale words
    # hold 4 column blocks); empty is a no-op
    assert lib.moe_pack_mx_weights(NULL, NULL, 4, 256, 96, NULL, NULL, NULL) == -3
    assert lib.moe_pack_mx_weights(NULL, NULL, 4, 200, 128, NULL, NULL, NULL) == -3
    assert lib.moe_pack_mx_weights(NULL, NULL, 4, 48, 128, NULL, NULL, NULL) == -3
    assert lib.moe_pack_mx_weights(NULL, NULL, 4, 192, 128, NULL, NULL, NULL) == -1
    assert lib.moe_pack_mx_weights(NULL, NULL, 0, 256, 128, NULL, NULL, NULL) == 0
    assert lib.moe_pack_mx_weights(NULL, NULL, 4, 256, 128, NULL, NULL, NULL) == -1
    # natural-weight GEMMs: the packed forms' checks
    assert lib.moe_grouped_gemm1_natural(NULL, NULL, NULL, 8, 128, 1152, 192, 128, NULL, NULL,
                                         NULL, NULL) == -3
    assert lib.moe_grouped_gemm2_natural(NULL, NULL, NULL, 8, 128, 1152, 256, 256, NULL, NULL,
                                         NULL, NULL) == -1
    assert lib.moe_grouped_gemm1_act_quant_natural(NULL, NULL, NULL, 8, 128, 1152, 256, 128,
                                                   NULL, NULL, ctypes.c_float(7.3), NULL, NULL,
                                                   NULL) == -5
    # fused group-128 GEMM1 + act-quant: I not a multiple of 128, a clamp
    # the sigma table does not cover, no output buffers
    g = lib.moe_grouped_gemm1_act_quant_g128
    assert g(NULL, NULL, NULL, 8, 128, 1152, 256, 200, NULL, NULL, ctypes.c_float(0.0), NULL, NULL,
             NULL) == -3
    assert g(NULL, NULL, NULL, 8, 128, 1152, 256, 128, NULL, NULL, ctypes.c_float(7.3), NULL, NULL,
             NULL) == -5
    assert g(NULL, NULL, NULL, 8, 128, 1152, 256, 128, NULL, NULL, ctypes.c_float(0.0), NULL, NULL,
             NULL) == -1
    # masked slab forms: m_pad not a multiple of 4, E_local * m_pad too
    # large, m_pad 0 with experts (scatter), then the aligned forms' checks
    ms = [NULL, 64, 2, 0, 8, 130, NULL, 256, NULL, NULL, NULL, NULL, NULL, 0, NULL]
    assert lib.moe_scatter_masked(*ms) == -3
    ms[5] = 1 << 28
    assert lib.moe_scatter_masked(*ms) == -2
    ms[5] = 0
    assert lib.moe_scatter_masked(*ms) == -2
    ms[5], ms[7] = 128, 200
    assert lib.moe_scatter_masked(*ms) == -3                                      # H % 128
    ms[7] = 256
    assert lib.moe_scatter_masked(*ms) == -1                                      # NULL pointers
    assert lib.moe_grouped_gemm1_masked(NULL, NULL, NULL, 8, 130, 256, 128, NULL, NULL, NULL,
                                        NULL) == -3
    assert lib.moe_grouped_gemm1_masked(NULL, NULL, NULL, 8, 128, 192, 128, NULL, NULL, NULL,
                                        NULL) == -3
    assert lib.moe_grouped_gemm1_masked(NULL, NULL, NULL, 8, 128, 256, 128, NULL, NULL, NULL,
                                        NULL) == -1
    assert lib.moe_grouped_gemm2_masked(NULL, NULL, NULL, 8, 128, 100, 256, NULL, NULL, NULL,
                                        NULL) == -3
    assert lib.moe_act_quant_masked(NULL, NULL, 8, 130, 128, ctypes.c_float(0.0), NULL, NULL,
                                    NULL) == -3
    assert lib.moe_act_quant_masked(NULL, NULL, 8, 128, 128, ctypes.c_float(7.3), NULL, NULL,
                                    NULL) == -5
    assert lib.moe_act_quant_masked(NULL, NULL, 8, 128, 128, ctypes.c_float(0.0), NULL, NULL,
                                    NULL) == -1
    assert lib.moe_grouped_gemm1_act_quant_masked(NULL, NULL, NULL, 8, 128, 256, 128, NULL, NULL,
                                                  ctypes.c_float(7.3), NULL, NULL, NULL) == -5
    assert lib.moe_grouped_gemm1_act_quant_masked(NULL, NULL, NULL, 8, 128, 256, 64, NULL, NULL,
                                                  ctypes.c_float(0.0), NULL, NULL, NULL) == -3
    assert lib.moe_grouped_gemm1_act_quant_masked(NULL, NULL, NULL, 8, 0, 256, 128, NULL, NULL,
                                                  ctypes.c_float(0.0), NULL, NULL, NULL) == 0
    # combine: H not a multiple of 8
    assert lib.moe_combine(NULL, 0, NULL, NULL, 4, 2, 12, ctypes.c_float(1.0), NULL, NULL) == -3
    # sparse GEMV: too many slots, unsupported format
    assert lib.moe_sparse_gemv(NULL, 0, NULL, 17, 4, 0, 32, 5760, 2880, 0, NULL, NULL, NULL, 1,
                               ctypes.c_float(1.702), ctypes.c_float(1.0), ctypes.c_float(7.0),
                               NULL, NULL, NULL) == -2
    assert lib.moe_sparse_gemv(NULL, 0, NULL, 1, 4, 0, 32, 5760, 2880, 3, NULL, NULL, NULL, 1,
                               ctypes.c_float(1.702), ctypes.c_float(1.0), ctypes.c_float(7.0),
                               NULL, NULL, NULL) == -5
    # GLU mode outside 0..2; GLU on load needs per-slot activation rows
    assert lib.moe_sparse_gemv(NULL, 1, NULL, 1, 4, 0, 32, 2880, 2880, 0, NULL, NULL, NULL, 3,
                               ctypes.c_float(1.702), ctypes.c_float(1.0), ctypes.c_float(7.0),
                               NULL, NULL, NULL) == -5
    assert lib.moe_sparse_gemv(NULL, 0, NULL, 1, 4, 0, 32, 2880, 2880, 0, NULL, NULL, NULL, 2,
                               ctypes.c_float(1.702), ctypes.c_float(1.0), ctypes.c_float(7.0),
                               NULL, NULL, NULL) == -5
    assert lib.moe_sparse_gemv(NULL, 1, NULL, 1, 4, 0, 32, 2880, 2880, 0, NULL, NULL, NULL, 2,
                               ctypes.c_float(1.702), ctypes.c_float(1.0), ctypes.c_float(7.0),
                               NULL, NULL, NULL) == -1


def test_hip_side_sigmoid_table_equals_oracle(tmp_path):
    """The HIP build's sigmoid table (own generator, long-double arithmetic)
    against the oracle's correctly rounded sigmoid, for every bf16 input."""
    from oracle import formats as F
    exe = tmp_path / "gen"
    src = os.path.join(ROOT, "mixture_experts_ffn_scatter_amd", "csrc", "gen_sigmoid_table.cpp")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-ffp-contract=off", src, "-o", str(exe)])
    txt = subprocess.check_output([str(exe)], text=True)
    lo = int(re.search(r"MOE_SIGMOID_EXP_LO (\d+)", txt).group(1))
    hi = int(re.search(r"MOE_SIGMOID_EXP_HI (\d+)", txt).group(1))
    tab = np.array([int(v, 16) for v in re.findall(r"0x([0-9a-f]{8})u", txt)], np.uint32)
    rows = hi - lo + 1
    assert tab.size == 2 * rows * 128
    b = np.arange(65536, dtype=np.uint32)
    ex = (b >> 7) & 0xFF
    finite = ex != 0xFF
    b, ex = b[finite], ex[finite]
    idx = (b >> 15) * rows * 128 + (np.clip(ex, lo, hi) - lo) * 128 + (b & 0x7F)
    want = F.sigmoid_f32(F.bf16_to_f32(b.astype(np.uint16))).view(np.uint32)
    assert np.array_equal(tab[idx], want)


def test_compact_sigmoid_lookup_equals_full_table(tmp_path):
    """The fused GEMM1 epilogue's compact sigmoid (rows 112..131 / 112..133 of
    the table, 1/2 + g/4 rounded with ties toward 1/2 below |g| = 2^-15, 1.0 /
    0.0 beyond the kept rows), restated here in the same IEEE operations,
    equals the full table's lookup for every bf16 pattern (inf and NaN
    included)."""
    exe = tmp_path / "gen"
    src = os.path.join(ROOT, "mixture_experts_ffn_scatter_amd", "csrc", "gen_sigmoid_table.cpp")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-ffp-contract=off", src, "-o", str(exe)])
    txt = subprocess.check_output([str(exe)], text=True)
    lo = int(re.search(r"MOE_SIGMOID_EXP_LO (\d+)", txt).group(1))
    hi = int(re.search(r"MOE_SIGMOID_EXP_HI (\d+)", txt).group(1))
    tab = np.array([int(v, 16) for v in re.findall(r"0x([0-9a-f]{8})u", txt)], np.uint32)
    rows = hi - lo + 1
    b = np.arange(65536, dtype=np.uint32)
    neg, ex, m = b >> 15, (b >> 7) & 0xFF, b & 0x7F
    full = tab[neg * rows * 128 + (np.clip(ex, lo, hi) - lo) * 128 + m]
    # the compact rule
    pos_lo, pos_hi, neg_lo, neg_hi = 112, 131, 112, 133
    g = (b << 16).view(np.float32)
    out = np.empty(65536, np.uint32)
    small = ex < pos_lo
    q = (g[small] * np.float32(0.25)).astype(np.float64)
    nudge = np.where(neg[small] == 1, 2.0 ** -50, -(2.0 ** -50))
    out[small] = (0.5 + q + nudge).astype(np.float32).view(np.uint32)
    p = (~small) & (neg == 0)
    out[p] = np.where(ex[p] > pos_hi, np.float32(1.0).view(np.uint32),
                      tab[(np.clip(ex[p], pos_lo, pos_hi) - lo) * 128 + m[p]])
    n = (~small) & (neg == 1)
    out[n] = np.where(ex[n] > neg_hi, np.uint32(0),
                      tab[rows * 128 + (np.clip(ex[n], neg_lo, neg_hi) - lo) * 128 + m[n]])
    bad = np.flatnonzero(out != full)
    assert bad.size == 0, f"{bad.size} patterns differ, first {[hex(v) for v in bad[:8]]}"


def test_division_free_scale_byte_equals_rounding_rule():
    """The kernels' UE8M0 byte taken straight from amax's bits when amax's
    exponent field is >= 10 (field minus 8, plus one when the mantissa field
    exceeds 0x600000, i.e. 1.m > 1.75; 0xFF for inf and 0 for NaN), restated
    here, equals the oracle's round-up rule on fl32(amax / 448) for every
    mantissa at exponent fields 10..12, 127 and 250..255. While amax and the
    quotient are normal (field >= 10), scaling amax by a power of two scales
    the rounded quotient by the same power, so these fields cover every
    case. Below field 10 the quotient is subnormal, its rounding can land on
    2^-127 from above (amax = 0x04600001 does), and the kernels divide."""
    from oracle import formats as F
    m = np.arange(1 << 23, dtype=np.uint32)
    for ex in [10, 11, 12, 127] + list(range(250, 256)):
        bits = (np.uint32(ex) << np.uint32(23)) | m
        amax = bits.view(np.float32)
        with np.errstate(invalid="ignore", over="ignore"):
            want = F.ue8m0_ceil_byte((amax / np.float32(448.0)).astype(np.float32))
        if ex == 255:
            got = np.where(m == 0, 0xFF, 0x00).astype(np.uint8)
        else:
            got = (ex - 8 + (m > 0x600000).astype(np.int64)).astype(np.uint8)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, f"exponent field {ex}: {bad.size} differ, first {hex(int(bits[bad[0]]))}"
    # the subnormal-quotient case the division is kept for
    q = np.array([0x04600001], np.uint32).view(np.float32) / np.float32(448.0)
    assert F.ue8m0_ceil_byte(q.astype(np.float32))[0] == 0


def test_hip_side_situ_tables_equal_oracle(tmp_path):
    """The HIP build's scaled-tanh tables (own generator, long double) with
    their identity / saturation rule outside the kept exponent rows, against
    the oracle's correctly rounded b * tanh(x / b), for every finite bf16."""
    from oracle import formats as F
    exe = tmp_path / "gen"
    src = os.path.join(ROOT, "mixture_experts_ffn_scatter_amd", "csrc", "gen_situ_table.cpp")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-ffp-contract=off", src, "-o", str(exe)])
    txt = subprocess.check_output([str(exe)], text=True)
    b = np.arange(65536, dtype=np.uint32)
    ex = (b >> 7) & 0xFF
    b = b[ex != 0xFF]
    ex = ex[ex != 0xFF]
    x = F.bf16_to_f32(b.astype(np.uint16)).astype(np.float32)
    for beta, name, macro in ((4.0, "g_tanh4_table", "TANH4"), (25.0, "g_tanh25_table", "TANH25")):
        lo = int(re.search(rf"MOE_{macro}_EXP_LO (\d+)", txt).group(1))
        hi = int(re.search(rf"MOE_{macro}_EXP_HI (\d+)", txt).group(1))
        body = txt.split(name)[1].split("};")[0]
        tab = np.array([int(v, 16) for v in re.findall(r"0x([0-9a-f]{8})u", body)], np.uint32)
        rows = hi - lo + 1
        assert tab.size == 2 * rows * 128
        got = np.where(ex < lo, x.view(np.uint32),
                       np.where(ex > hi, np.where(b >> 15, np.float32(-beta), np.float32(beta)).view(np.uint32),
                                tab[(b >> 15) * rows * 128 + (np.clip(ex, lo, hi) - lo) * 128 + (b & 0x7F)]))
        want = F.scaled_tanh_f32(x, beta).view(np.uint32)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, f"beta {beta}: {bad.size} differ, first bf16 {[hex(int(v)) for v in b[bad[:4]]]}"
