"""lora_proj_noalloc, the entry point that allocates nothing, through the C-ABI: two calls in a
row, the second with a smaller input, each bitwise equal to lora_proj's result on the same
inputs (the same kernels run; only the workspace differs); a decode call after a prefill call
sees clean counters; the random sweep's shapes and tables back to back on the one array; a call
whose scratch would exceed the fixed array is refused."""
from __future__ import annotations

import numpy as np
import pytest

import gates
from gpu_util import log, to_device, y_bits, y_to_numpy
from oracle import lora_proj_ref
from rank_adapted_gemm_amd import binding as bd
from rank_adapted_gemm_amd import synth

pytestmark = pytest.mark.gpu

CALLS = [
    # a prefill call (shrink + output kernel, T in the array), then a smaller decode call (counters,
    # partial sums and T in the array)
    dict(M=300, N=1000, K=520, rank=32, seg_starts=[0, 40, 300], seg_adapter=[-1, 0], scale=0.5),
    dict(M=70, N=520, K=200, rank=48, seg_starts=[0, 64, 70], seg_adapter=[0, -1], scale=1.0),
]


def test_noalloc_equals_lora_proj_on_two_calls():
    import torch
    for i, c in enumerate(CALLS):
        p = synth.random_problem(95 + i, **c)
        log(f"case noalloc call {i} M={p.M} path={bd.path(p.M, p.N, p.K, p.rank)}")
        X, W, A, B = to_device(p)
        ref = bd.lora_proj(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale)
        out = torch.empty((p.M, p.N), dtype=torch.bfloat16, device="cuda")
        y = bd.lora_proj_noalloc(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale, out)
        torch.cuda.synchronize()
        assert np.array_equal(y_bits(y), y_bits(ref))
        assert gates.passes_bf16(y_to_numpy(y), lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B,
                                                              p.scale))


def test_noalloc_split_shrink():
    """A prefill call whose shrink splits over K (4 splits: its fp32 partials sit in the array after
    T), then a call that does not split: each bitwise equal to lora_proj."""
    import torch
    calls = [dict(M=300, N=520, K=2056, rank=48, seg_starts=[0, 40, 41, 200, 300], seg_adapter=[0, -1, 1, 0],
                  n_adapters=2, scale=0.5),
             dict(CALLS[0])]
    for i, c in enumerate(calls):
        p = synth.random_problem(98 + i, **c)
        log(f"case noalloc split call {i} M={p.M} K={p.K}")
        X, W, A, B = to_device(p)
        ref = bd.lora_proj(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale)
        out = torch.empty((p.M, p.N), dtype=torch.bfloat16, device="cuda")
        y = bd.lora_proj_noalloc(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale, out)
        torch.cuda.synchronize()
        assert np.array_equal(y_bits(y), y_bits(ref))


def test_noalloc_repeated_decode_calls_stay_exact():
    """Integer inputs: several decode calls in a row on the one array (each clears its counters),
    every one exact."""
    import torch
    p = synth.random_problem(97, integer=True, **dict(CALLS[1], scale=1.0))
    exact = lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale)
    X, W, A, B = to_device(p)
    out = torch.empty((p.M, p.N), dtype=torch.float32, device="cuda")
    for _ in range(3):
        out.fill_(float("nan"))
        bd.lora_proj_noalloc(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale, out, dtype="bf16_f32out")
        torch.cuda.synchronize()
        assert np.array_equal(y_to_numpy(out), exact)


def test_noalloc_random_calls_in_a_row():
    """The random sweep's shapes and segment tables (one rank, the largest of each call's, and one
    scale; no slices, which this entry point does not take) back to back on the one array, decode
    and prefill calls of every size in turn: each bitwise equal to lora_proj on the same inputs."""
    import torch
    from test_gpu_random_shapes import N_CASES, case
    ran = 0
    for i in range(N_CASES):
        c = case(i)
        N = sum(c["widths"]) if c["widths"] else c["N"]
        r, n_ad = max(c["ranks"]), len(c["ranks"])
        if bd.workspace_bytes(c["M"], N, c["K"], r, n_ad) > bd.NOALLOC_SCRATCH_BYTES:
            continue
        p = synth.random_problem(9600 + i, M=c["M"], N=N, K=c["K"], rank=r, n_adapters=n_ad, scale=0.75,
                                 seg_starts=c["seg_starts"], seg_adapter=c["seg_adapter"])
        log(f"case noalloc random {i} M={p.M} N={N} K={p.K} r={r} path={bd.path(p.M, N, p.K, r)}")
        X, W, A, B = to_device(p)
        ref = bd.lora_proj(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale)
        out = torch.full((p.M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        y = bd.lora_proj_noalloc(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale, out)
        torch.cuda.synchronize()
        assert np.array_equal(y_bits(y), y_bits(ref)), i
        ran += 1
    assert ran >= 80, ran


def test_noalloc_refuses_scratch_past_the_array():
    """T of 70,000 rows at rank 512 (143 MB) does not fit the 64 MiB array: LORA_EWORKSPACE before
    any launch (the addresses are never touched, so stand-ins serve)."""
    fake = 1 << 40
    M, N, K, r = 70000, 256, 64, 512
    assert bd.workspace_bytes(M, N, K, r, 1) > bd.NOALLOC_SCRATCH_BYTES
    st = bd.lora_proj_noalloc_raw(fake, [0, M], [0], fake + (1 << 34), [fake + (2 << 34)], [fake + (3 << 34)], r,
                                  1.0, fake + (4 << 34), M, N, K, "bf16")
    assert st == bd.LORA_EWORKSPACE
