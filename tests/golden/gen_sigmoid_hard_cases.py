"""Writes sigmoid_hard_cases.txt: every fp32 input v in (-110, 110) whose
sigmoid 1/(1+e^-v), evaluated in fp64, lies within 2^-45 (relative) of a
rounding midpoint between two fp32 values -- the inputs where an fp64
evaluation alone cannot be trusted to give the correctly rounded fp32 value
-- with that correctly rounded value from the oracle's decimal evaluation.

Screening runs over all 2.2e9 fp32 values of the range in fp64 with numpy
(a few minutes); the expected values come from oracle.formats only.
Run from the repository root: python tests/golden/gen_sigmoid_hard_cases.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle.formats import _decimal_to_f32_rne, sigmoid_exact_decimal  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sigmoid_hard_cases.txt")
CHUNK = 1 << 24


def screen(bits: np.ndarray) -> np.ndarray:
    v = bits.view(np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-v))
    f = s.astype(np.float32)
    fd = f.astype(np.float64)
    lo = np.nextafter(f, np.float32(-np.inf)).astype(np.float64)
    hi = np.nextafter(f, np.float32(np.inf)).astype(np.float64)
    margin = np.minimum(np.abs(s - 0.5 * (fd + lo)), np.abs(s - 0.5 * (fd + hi)))
    return bits[margin <= 2.0 ** -45 * s]


def main():
    top = int(np.float32(110.0).view(np.uint32))
    found = []
    for sign in (0, 0x80000000):
        for b0 in range(0, top, CHUNK):
            bits = np.arange(b0, min(b0 + CHUNK, top), dtype=np.uint32) | np.uint32(sign)
            found.append(screen(bits))
        print(f"sign {sign:#x} done, {sum(a.size for a in found)} candidates", flush=True)
    cand = np.unique(np.concatenate(found))
    lines = []
    for b in cand:
        v = float(np.uint32(b).view(np.float32))
        want = _decimal_to_f32_rne(sigmoid_exact_decimal(v, prec=80))
        lines.append(f"{int(b):08x} {int(np.float32(want).view(np.uint32)):08x}")
    with open(OUT, "w") as fh:
        fh.write("# fp32 inputs v in (-110, 110) whose fp64 sigmoid lies within 2^-45 of an fp32\n")
        fh.write("# rounding midpoint, and the correctly rounded fp32 sigmoid of each (80-digit\n")
        fh.write("# decimal evaluation, ties to even). Written by gen_sigmoid_hard_cases.py.\n")
        fh.write("# columns: bits of v, bits of round_fp32(1/(1+exp(-v)))\n")
        fh.write("\n".join(lines) + "\n")
    print(f"{len(lines)} cases -> {OUT}")


if __name__ == "__main__":
    main()
