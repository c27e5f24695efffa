"""Helpers for GPU tests: move a synthetic problem to the device, call the C-ABI, read back."""
from __future__ import annotations

import json
import os
import sys

import numpy as np

from rank_adapted_gemm_amd import binding as bd
from rank_adapted_gemm_amd import synth


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def record(case: str, rep: dict, past_g1: int):
    """Append one parity result (rms, G1, G2, elements past the literal G1 bound) to the JSON-lines
    file named by LORA_PARITY_RECORD, when set, so the figures of every large case are kept."""
    path = os.environ.get("LORA_PARITY_RECORD")
    if not path:
        return
    with open(path, "a") as f:
        f.write(json.dumps(dict(case=case, rms=rep["rms"], g1=rep["g1"], g2=rep["g2"], past_g1=int(past_g1))) + "\n")


def _dev_bf16(bits, torch, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def to_device(p: synth.Problem, dev="cuda"):
    """(X, W, A list, B list) as device tensors of the problem's input dtype."""
    import torch
    if p.dtype == "f32":
        f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
        return f(p.X), f(p.W), [f(a) for a in p.A], [f(b) for b in p.B]
    if p.X_bits is None:
        raise ValueError("bf16 problem without bf16 bits")
    return (_dev_bf16(p.X_bits, torch, dev), _dev_bf16(p.W_bits, torch, dev),
            [_dev_bf16(a, torch, dev) for a in p.A_bits], [_dev_bf16(b, torch, dev) for b in p.B_bits])


def y_to_numpy(y):
    """float64 values of a device output (bf16 or fp32)."""
    import torch
    if y.dtype == torch.bfloat16:
        bits = y.view(torch.int16).cpu().numpy().view(np.uint16)
        return synth.bf16_bits_to_f32(bits).astype(np.float64)
    return y.float().cpu().numpy().astype(np.float64)


def y_bits(y):
    import torch
    return y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run(p: synth.Problem, dtype=None, scale=None, seg_adapter=None, dev_inputs=None):
    """Run the HIP path on problem p and return the device output tensor."""
    import torch
    dtype = dtype or p.dtype
    X, W, A, B = dev_inputs if dev_inputs is not None else to_device(p)
    y = bd.lora_proj(X, list(p.seg_starts), list(p.seg_adapter if seg_adapter is None else seg_adapter),
                     W, A, B, p.scale if scale is None else scale, dtype=dtype)
    torch.cuda.synchronize()
    return y
