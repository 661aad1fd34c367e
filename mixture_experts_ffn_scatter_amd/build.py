"""Build the gfx950 HIP library ``libmoe_ffn.so`` in-tree.

Steps: compile and run the host generators of the sigmoid and SiTU tables, compile
every ``csrc/*.hip`` with hipcc for gfx950 (in parallel), link one shared
library next to this file. Run ``python -m mixture_experts_ffn_scatter_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
GEN = os.path.join(BUILD, "gen")
LIB = os.path.join(HERE, "libmoe_ffn.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",                     # no silent fused multiply-adds
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout)
        raise RuntimeError(f"build step failed: {cmd[0]}")
    return r.stdout


def generate_tables():
    """The sigmoid table and the SiTU scaled-tanh tables, from their host
    generators (long double; each checks its own rounding margins)."""
    os.makedirs(GEN, exist_ok=True)
    for gen, inc in (("gen_sigmoid_table", "sigmoid_table.inc"), ("gen_situ_table", "situ_table.inc")):
        exe = os.path.join(BUILD, gen)
        _run(["g++", "-O2", "-std=c++17", "-ffp-contract=off",
              os.path.join(CSRC, gen + ".cpp"), "-o", exe])
        out = _run([exe])
        path = os.path.join(GEN, inc)
        with open(path + ".tmp", "w") as f:
            f.write(out)
        os.replace(path + ".tmp", path)


def compile_one(src):
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))
    _run([HIPCC, *HIP_FLAGS, "-I", GEN, "-c", src, "-o", obj])
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    generate_tables()
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
