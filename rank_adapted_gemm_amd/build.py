"""Builds liblora_proj.so (the C-ABI library with the gfx950 kernels) in-tree.

    python -m rank_adapted_gemm_amd.build            # compile
    python -m rank_adapted_gemm_amd.build --report   # also print per-kernel register/LDS use
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "liblora_proj.so"
SOURCES = ["lora_api.cpp", "lora_bf16.hip", "lora_decode.hip", "lora_f32.hip", "lora_q4.hip", "lora_extract.hip",
           "lora_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the kernels)")


def flags(report: bool = False) -> list[str]:
    f = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         # no packed fp32 arithmetic anywhere in the device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
    if report:
        f.append("-Rpass-analysis=kernel-resource-usage")
    return f


def build(report: bool = False, verbose: bool = False) -> str:
    out = os.path.join(PKG, LIB_NAME)
    tmp = out + ".tmp"
    cmd = [hipcc(), *flags(report), "-shared", "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if msgs.strip() and (verbose or report):
        print(msgs, flush=True)
    os.replace(tmp, out)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--report", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    path = build(report=a.report, verbose=a.verbose)
    print(path)


if __name__ == "__main__":
    sys.exit(main())
