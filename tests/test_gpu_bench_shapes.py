"""Parity at the exact shapes the benchmark times, and the negative controls at two workloads.

Each case here uses the host recipe's draws (synth) for inputs of the same shape, segment table
and adapter count as a bench line, so the kernels run with the same launch plan that bench.py
times; the oracle is the fp64 definition.

  * suffix decode, grouped: q/k/v as one sliced call (15,360 x 5,120) and gate/up as one
    (34,816 x 5,120), M = 70 (64 adapter rows + 6 base rows), every element; the same two calls
    with 4-bit base weights.
  * prefill16k with four adapters: 212 segments of 20-140 rows over 16,384 rows, q, gate and
    down, sampled rows.
  * negative controls (the pages' red-arm idea: a deliberately broken variant must fail): adapter
    off, s doubled, A passed untransposed, B passed transposed, X rows shifted by one, a segment
    boundary off by one, base rows given the adapter; at the tiny case (fp32 test mode) and at
    the mixed batch (6 decode rows around a 2,048-row chunk, bf16).
"""
from __future__ import annotations

import numpy as np
import pytest

import gates
from gpu_util import log, record, to_device, y_to_numpy
from oracle import lora_proj_q4_ref, lora_proj_ref, lora_proj_sliced_ref
from rank_adapted_gemm_amd import binding as bd
from rank_adapted_gemm_amd import synth

pytestmark = pytest.mark.gpu


def _dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def grouped_problem(name, members):
    """A suffix layer-0 group (members: projection indices) as one sliced problem: W stacked along
    N, each A stacked by slice, B stacked along N (the bench's group_layer on host draws)."""
    w = synth.WORKLOADS["suffix"]
    shapes = synth.projections("suffix")
    K = shapes[members[0]][1]
    x = synth.layer_input(w["cfg"], 0, w["M"], K)
    Wb, Wf, Ab, Af, Bb, Bf, widths = [], [], [], [], [], [], []
    for j in members:
        _, Kj, N = shapes[j]
        assert Kj == K
        (wb, wf), (ab, af), (bb, bf) = synth.projection_weights(w["cfg"], 0, j, K, N)
        Wb.append(wb), Wf.append(wf), Ab.append(ab), Af.append(af), Bb.append(bb), Bf.append(bf)
        widths.append(N)
    cat = lambda xs: np.ascontiguousarray(np.concatenate(xs, axis=0))
    p = synth.Problem(X=x[1], W=cat(Wf), A=[cat(Af)], B=[cat(Bf)],
                      seg_starts=np.array(w["seg_starts"], np.int32), seg_adapter=np.array(w["seg_adapter"], np.int32),
                      scale=[w["scale"]], dtype="bf16", X_bits=x[0], W_bits=cat(Wb), A_bits=[cat(Ab)],
                      B_bits=[cat(Bb)], name=f"suffix/L0/{name}")
    return p, widths


GROUPS = {"qkv": (0, 1, 2), "gate_up": (4, 5)}


def check(p, y, ref, literal=True):
    rep = gates.report(y, ref)
    over = np.abs(y - ref) > gates.BF16_TOL * rep["rms"]
    log(f"  {p.name} rms={rep['rms']:.4g} G1={rep['g1']:.3e} G2={rep['g2']:.3e} past-G1={int(over.sum())}")
    record(p.name, rep, int(over.sum()))
    assert rep["nonfinite"] == 0 and rep["g2"] <= gates.BF16_TOL, rep
    if over.any():
        assert not literal, rep
        assert gates.explained_by_rounding(y[over], ref[over], rep["rms"]).all()


@pytest.mark.parametrize("group", list(GROUPS))
def test_suffix_grouped_bf16_full(group):
    """The grouped decode line's sliced calls at their timed shapes, every element."""
    import torch
    p, widths = grouped_problem(group, GROUPS[group])
    log(f"case grouped decode {group} N={p.N} K={p.K} slices={widths} path={bd.path(p.M, p.N, p.K, 256)}")
    assert bd.path(p.M, p.N, p.K, 256) == "decode"
    X, W, A, B = to_device(p)
    y = bd.lora_proj(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale, slices=widths)
    torch.cuda.synchronize()
    ref = lora_proj_sliced_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale, widths)
    check(p, y_to_numpy(y), ref)


@pytest.mark.parametrize("group", list(GROUPS))
def test_suffix_grouped_q4_full(group):
    """The 4-bit grouped decode line's sliced calls at their timed shapes, every element, against
    the oracle's exact dequantized weights."""
    import torch
    p, widths = grouped_problem(group, GROUPS[group])
    p.name += " q4"
    packed, params, *_ = synth.quantize_q4(p.W)
    log(f"case grouped q4 decode {group} N={p.N} K={p.K} slices={widths}")
    X, _, A, B = to_device(p)
    Wq = torch.from_numpy(packed).to("cuda")
    Wp = torch.from_numpy(np.ascontiguousarray(params).view(np.int32)).to("cuda")
    y = bd.lora_proj_q4(X, list(p.seg_starts), list(p.seg_adapter), Wq, Wp, A, B, p.scale, slices=widths)
    torch.cuda.synchronize()
    ref = lora_proj_q4_ref(p.X, p.seg_starts, p.seg_adapter, packed, params, p.A, p.B, p.scale, slice_n=widths)
    check(p, y_to_numpy(y), ref)


@pytest.mark.parametrize("proj", [0, 4, 6])
def test_prefill16k_four_adapters_sampled(proj):
    """The many-adapters prefill line at its timed shape: 16,384 rows in 212 seeded segments, each
    naming one of four adapters or none; sampled rows (every segment's first and last row)."""
    import torch
    w = synth.WORKLOADS["prefill16k"]
    cfg, M = w["cfg"], w["M"]
    name, K, N = synth.PROJECTIONS[proj]
    starts, labels = synth.mixed_table(M)
    assert len(labels) == 212
    x = synth.layer_input(cfg, 0, M, K)
    (Wb, Wf), (Ab, Af), (Bb, Bf) = synth.projection_weights(cfg, 0, proj, K, N)
    A_bits, A_vals, B_bits, B_vals = [Ab], [Af], [Bb], [Bf]
    for j in range(1, synth.MIXED_ADAPTERS):
        ab, af = synth.normal_bf16(synth.extra_adapter_seed(cfg, 0, proj, synth.T_A, j), (synth.RANK, K),
                                   synth.SIGMA_WAB)
        bb, bf = synth.normal_bf16(synth.extra_adapter_seed(cfg, 0, proj, synth.T_B, j), (N, synth.RANK),
                                   synth.SIGMA_WAB)
        A_bits.append(ab), A_vals.append(af), B_bits.append(bb), B_vals.append(bf)
    log(f"case prefill16k four adapters proj={name} segments={len(labels)}")
    y = bd.lora_proj(_dev_bf16(x[0]), starts, labels, _dev_bf16(Wb), [_dev_bf16(a) for a in A_bits],
                     [_dev_bf16(b) for b in B_bits], 1.0)
    torch.cuda.synchronize()
    rows = synth.sample_rows(M, starts, 512, seed=500 + proj)
    ref = lora_proj_ref(x[1], starts, labels, Wf, A_vals, B_vals, 1.0, rows=rows)
    p = synth.Problem(X=x[1], W=Wf, A=A_vals, B=B_vals, seg_starts=np.array(starts), seg_adapter=np.array(labels),
                      scale=1.0, dtype="bf16", name=f"prefill16k 4 adapters {name}")
    check(p, y_to_numpy(y)[rows], ref, literal=False)


# ------------------------------------------------------------------ negative controls
ARMS = ["adapter_off", "scale_doubled", "A_untransposed", "B_transposed", "X_rows_shifted",
        "boundary_off_by_one", "base_rows_given_adapter"]


def broken_call(p, arm, dev):
    """Run the kernels on a deliberately wrong version of problem p's call."""
    import torch
    X, W, A, B = dev
    starts, labels, scale = list(p.seg_starts), list(p.seg_adapter), p.scale
    r, K, N = p.rank, p.K, p.N
    if arm == "adapter_off":
        labels = [-1] * len(labels)
    elif arm == "scale_doubled":
        scale = 2 * scale
    elif arm == "A_untransposed":      # the K x r transpose's bytes read as r x K
        A = [a.t().contiguous().view(r, K) for a in A]
    elif arm == "B_transposed":        # the r x N transpose's bytes read as N x r
        B = [b.t().contiguous().view(N, r) for b in B]
    elif arm == "X_rows_shifted":
        X = torch.roll(X, 1, dims=0).contiguous()
    elif arm == "boundary_off_by_one":   # the first adapter segment starts one row later
        g = next(i for i, a in enumerate(labels) if a >= 0)
        starts[g] += 1
        assert starts[g] <= starts[g + 1]
    elif arm == "base_rows_given_adapter":
        labels = [0] * len(labels)
    y = bd.lora_proj(X, starts, labels, W, A, B, scale, dtype=p.dtype)
    torch.cuda.synchronize()
    return y_to_numpy(y)


@pytest.fixture(scope="module")
def arm_cases():
    cache = {}

    def get(name):
        if name not in cache:
            if name == "tiny":
                p = synth.tiny()
            else:
                p = synth.workload_problem("mixed", proj=0)
            ref = lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale)
            cache[name] = (p, ref, to_device(p))
        return cache[name]
    return get


@pytest.mark.parametrize("case", ["tiny", "mixed"])
@pytest.mark.parametrize("arm", ARMS)
def test_negative_control_arms(arm_cases, case, arm):
    """Each broken variant fails the gate of its case (fp32 test mode at tiny, G2 at mixed), while
    the unbroken call passes it."""
    p, ref, dev = arm_cases(case)
    log(f"case red arm {arm} at {case}")
    passes = gates.passes_f32 if p.dtype == "f32" else gates.passes_bf16
    y = broken_call(p, arm, dev)
    assert not passes(y, ref), f"{arm} at {case} passed the gate"
    if arm == ARMS[0]:   # once per case: the real call passes
        import torch
        X, W, A, B = dev
        good = bd.lora_proj(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale, dtype=p.dtype)
        torch.cuda.synchronize()
        assert passes(y_to_numpy(good), ref)
