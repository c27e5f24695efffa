"""Builds liblora_proj.so (the C-ABI library with the gfx950 kernels) in-tree.

    python -m rank_adapted_gemm_amd.build            # compile
    python -m rank_adapted_gemm_amd.build --report   # also print per-kernel register/LDS use
"""
from __future__ import annotations

import argparse
import concurrent.futures
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


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    return res.returncode, msgs


def build(report: bool = False, verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source to an object file (in parallel, under _build/), then link the library."""
    out = os.path.join(PKG, LIB_NAME)
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    cmds = [[hipcc(), *flags(report), "-c", "-o", os.path.join(objdir, s + ".o"), os.path.join(CSRC, s)]
            for s in SOURCES]
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    for (rc, msgs), src in zip(results, SOURCES):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{msgs}")
        if msgs.strip() and (verbose or report):
            print(msgs, flush=True)
    tmp = out + ".tmp"
    rc, msgs = _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", tmp,
                     *[os.path.join(objdir, s + ".o") for s in SOURCES]], verbose)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{msgs}")
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
