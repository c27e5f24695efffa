"""Adapters of different ranks in one call (lora_proj_ranked), through the C-ABI.

Each adapter's factors are stored compact at its own rank (A_a (S r_a) x K, B_a N x r_a); the oracle
takes each adapter at its own rank too.  Covered on every kernel path: prefill (several adapters of
ranks 16, 48, 256 and 32 inside one row tile), decode (the A blocks' T and the expand units past a
smaller adapter's rank), sliced calls on both paths, the fp32 test mode, and equality with the same
call made through lora_proj_sliced with every adapter zero-padded to the largest rank."""
from __future__ import annotations

import numpy as np
import pytest

import gates
from gpu_util import log, record, to_device, y_to_numpy
from oracle import lora_proj_ref, lora_proj_sliced_ref
from rank_adapted_gemm_amd import binding as bd
from rank_adapted_gemm_amd import synth

pytestmark = pytest.mark.gpu

PREFILL = dict(M=700, N=520, K=264, seg_starts=[0, 40, 41, 200, 230, 260, 300, 512, 700],
               seg_adapter=[2, -1, 0, 1, 3, 2, -1, 1])
DECODE = dict(M=70, N=1000, K=520, seg_starts=[0, 20, 21, 50, 64, 70], seg_adapter=[1, -1, 0, 2, -1])
RANKS4 = [16, 48, 256, 32]
SCALES4 = [1.0, 0.5, -2.0, 0.25]
RANKS3 = [32, 128, 64]
SCALES3 = [0.5, 1.0, -1.0]


def ranked_problem(seed, case, ranks, scales, integer, slices=None, dtype="bf16"):
    c = dict(case)
    if slices is not None:
        c["N"] = sum(slices)
    return synth.random_problem(seed, rank=16, n_adapters=len(ranks), ranks=ranks, scale=list(scales),
                                integer=integer, dtype=dtype, slices=1 if slices is None else len(slices), **c)


def oracle(p, slices=None):
    if slices is None:
        return lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale)
    return lora_proj_sliced_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale, slices)


def run(p, dtype, slices=None):
    import torch
    X, W, A, B = to_device(p)
    y = bd.lora_proj_ranked(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale, dtype=dtype,
                            slices=slices)
    torch.cuda.synchronize()
    return y


CASES = {
    "prefill": (PREFILL, RANKS4, SCALES4, None),
    "decode": (DECODE, RANKS3, SCALES3, None),
    "prefill_sliced": (dict(PREFILL, N=None), [48, 16, 32, 256], SCALES4, [256, 512, 256]),
    "decode_sliced": (dict(DECODE, N=None), [16, 64, 32], SCALES3, [256, 256, 512]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_ranked_exact(name):
    """Integer inputs: the fp32 store equals the exact result bit for bit and the bf16 store is its
    correct rounding."""
    case, ranks, scales, slices = CASES[name]
    p = ranked_problem(51, case, ranks, scales, integer=True, slices=slices)
    log(f"case ranked exact {name} path={bd.path(p.M, p.N, p.K, max(ranks))} ranks={ranks}")
    exact = oracle(p, slices)
    y32 = y_to_numpy(run(p, "bf16_f32out", slices))
    bad = np.argwhere(y32 != exact)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    y16 = y_to_numpy(run(p, "bf16", slices))
    want = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(exact.astype(np.float32))).astype(np.float64)
    assert np.array_equal(y16, want)


@pytest.mark.parametrize("name", list(CASES))
def test_ranked_equals_zero_padded(name):
    """Gaussian inputs: the ranked call against the oracle at the G2 bar, and against lora_proj_sliced
    with every adapter zero-padded to the largest rank (the padded terms add exact zeros, so the two
    agree to the value; only the sign of an exact zero may differ)."""
    import torch
    case, ranks, scales, slices = CASES[name]
    p = ranked_problem(52, case, ranks, scales, integer=False, slices=slices)
    widths = slices if slices is not None else [p.N]
    S, R = len(widths), max(ranks)
    y = run(p, "bf16", slices)
    ref = oracle(p, slices)
    yn = y_to_numpy(y)
    rep = gates.report(yn, ref)
    over = np.abs(yn - ref) > gates.BF16_TOL * rep["rms"]
    log(f"  ranked {name} rms={rep['rms']:.4g} G1={rep['g1']:.3e} G2={rep['g2']:.3e} past-G1={int(over.sum())}")
    record(f"ranked/{name}", rep, int(over.sum()))
    assert rep["nonfinite"] == 0 and rep["g2"] <= gates.BF16_TOL, rep
    # the adapter of scale -2 gives some rows outputs far above the rms, where half
    # a bf16 ulp alone passes the literal bound: those must be correct roundings
    if over.any():
        assert gates.explained_by_rounding(yn[over], ref[over], rep["rms"]).all()
    X, W, A, B = to_device(p)
    Ap, Bp = [], []
    for a, b, r in zip(A, B, ranks):
        ap = torch.zeros((S * R, p.K), dtype=a.dtype, device=a.device)
        for s in range(S):
            ap[s * R:s * R + r] = a[s * r:(s + 1) * r]
        bp = torch.zeros((p.N, R), dtype=b.dtype, device=b.device)
        bp[:, :r] = b
        Ap.append(ap.contiguous())
        Bp.append(bp.contiguous())
    y_pad = bd.lora_proj(X, list(p.seg_starts), list(p.seg_adapter), W, Ap, Bp, list(scales), slices=widths)
    torch.cuda.synchronize()
    assert np.array_equal(y_to_numpy(y), y_to_numpy(y_pad))


def test_ranked_fp32_test_mode():
    """fp32 inputs and arithmetic, mixed ranks on the prefill shape: <= 1e-5 rms."""
    p = ranked_problem(53, PREFILL, RANKS4, SCALES4, integer=False, dtype="f32")
    y = y_to_numpy(run(p, "f32"))
    assert gates.passes_f32(y, oracle(p))


def test_ranked_on_a_shared_workspace():
    """Prefill then decode calls of different rank mixes on one workspace sized for the largest:
    each exact (the decode counters left at zero by each call)."""
    import torch
    ws = torch.zeros(max(bd.workspace_bytes(700, 520, 264, 256, 4), bd.workspace_bytes(70, 1000, 520, 128, 3)),
                     dtype=torch.uint8, device="cuda")
    for i, (case, ranks, scales) in enumerate(((DECODE, RANKS3, SCALES3), (PREFILL, RANKS4, SCALES4),
                                               (DECODE, [16, 16, 128], SCALES3))):
        p = ranked_problem(60 + i, case, ranks, scales, integer=True)
        X, W, A, B = to_device(p)
        y = bd.lora_proj_ranked(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale, workspace=ws,
                                dtype="bf16_f32out")
        torch.cuda.synchronize()
        assert np.array_equal(y_to_numpy(y), oracle(p))
    assert bd.workspace_status(ws) == bd.LORA_OK
