"""Writes tiny_oracle.txt: values of the fp64 oracle on the 64x256 fp32 case.

Calls only the oracle and the seeded input generator.  Run from the repository
root: python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import lora_proj_ref  # noqa: E402
from rank_adapted_gemm_amd import synth  # noqa: E402


def main():
    p = synth.tiny()
    y = lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale)
    g = np.random.Generator(np.random.PCG64(2024))
    picks = [(0, 0), (31, 511), (32, 0), (63, 511)] + [
        (int(m), int(n)) for m, n in zip(g.integers(0, 64, 28), g.integers(0, 512, 28))]
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.txt")
    with open(out, "w") as f:
        f.write("# fp64 oracle on the tiny case (X 64x256, W 512x256, rank 16, s = 0.5, seed 0;\n")
        f.write("# rows 0-31 base-only, 32-63 adapter).  Written by tests/golden/make_golden.py.\n")
        f.write(f"rms_base_rows {np.sqrt(np.mean(y[:32] ** 2)):.17g}\n")
        f.write(f"rms_adapter_rows {np.sqrt(np.mean(y[32:] ** 2)):.17g}\n")
        for m, n in picks:
            f.write(f"y[{m},{n}] {y[m, n]:.17g}\n")


if __name__ == "__main__":
    main()
