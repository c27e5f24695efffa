"""The decode kernel's hand-overs between blocks, through the C-ABI: a lost hand-over is never
silent.  Its outputs hold NaN and lora_workspace_status reports it (and restores the counter
area).  The failures are forced from the host: a counter area pre-filled with counts past every
total (so every wait passes at once), and the library's test hook, which makes every wait for T
give up after a short bounded spin.  Every block still exits normally in both."""
from __future__ import annotations

import numpy as np
import pytest

import gates
from gpu_util import log, to_device, y_to_numpy
from oracle import lora_proj_ref
from rank_adapted_gemm_amd import binding as bd
from rank_adapted_gemm_amd import synth

pytestmark = pytest.mark.gpu

C = bd.WORKSPACE_COUNTER_BYTES
CASES = {
    # several blocks share each 128-row weight tile: partial sums handed to the tile's last block
    "shared_tiles": dict(M=70, N=520, K=200, rank=48, seg_starts=[0, 30, 64, 70], seg_adapter=[1, 0, -1],
                         n_adapters=2),
    # K = 64: one unit per tile, so most blocks cover whole tiles and run past them
    "whole_tiles": dict(M=70, N=40960, K=64, rank=32, seg_starts=[0, 64, 70], seg_adapter=[0, -1], n_adapters=1),
}


def workspace_for(p):
    import torch
    need = bd.workspace_bytes(p.M, p.N, p.K, p.rank, len(p.A))
    return torch.zeros(need, dtype=torch.uint8, device="cuda")


def call(p, ws, dtype="bf16", seg_adapter=None):
    import torch
    X, W, A, B = to_device(p)
    y = bd.lora_proj(X, list(p.seg_starts), list(p.seg_adapter if seg_adapter is None else seg_adapter), W, A, B,
                     p.scale, workspace=ws, dtype=dtype)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("name", list(CASES))
def test_plan_of_case(name):
    c = CASES[name]
    plan = bd.decode_plan(c["M"], c["N"], c["K"], c["rank"], c["n_adapters"])
    units = plan["ntW"] * plan["nst"]
    if name == "whole_tiles":
        assert units > plan["GW"]              # a block's range spans more than one tile
    else:
        assert plan["smaxW"] >= 2              # tiles shared between blocks


@pytest.mark.parametrize("name", list(CASES))
def test_stale_counts_are_reported(name):
    """A counter area left non-zero, here every count past any total (as a call that never
    finished could leave it): every wait passes at once and every block exits normally, every
    tile's arrivals find its count past the total and store NaN over the tile, the status query
    reports LORA_EHANDOVER and restores the area, and the next call on the workspace is exact."""
    import torch
    p = synth.random_problem(71, integer=True, scale=[1.0, 0.5][:CASES[name]["n_adapters"]], **CASES[name])
    log(f"case stale counters {name} plan={bd.decode_plan(p.M, p.N, p.K, p.rank, len(p.A))}")
    exact = lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale)
    ws = workspace_for(p)
    ws[:C - 8].view(torch.int64).fill_(1000)
    y_bad = y_to_numpy(call(p, ws, dtype="bf16_f32out"))
    assert np.isnan(y_bad).all()
    assert bd.workspace_status(ws) == bd.LORA_EHANDOVER
    assert int(torch.count_nonzero(ws[:C])) == 0          # the query restored the counter area
    y = y_to_numpy(call(p, ws, dtype="bf16_f32out"))
    bad = np.argwhere(y != exact)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    assert bd.workspace_status(ws) == bd.LORA_OK


@pytest.mark.parametrize("name", list(CASES))
def test_lost_handover_is_reported_and_poisons_output(name):
    """With the test hook on, every wait for T gives up: the call's output is NaN wherever it
    depended on T (every column: every weight tile adds an expand), the status query reports
    LORA_EHANDOVER once and clears it, and the next normal call on the same workspace is
    correct."""
    p = synth.random_problem(72, scale=[0.5, 1.0][:CASES[name]["n_adapters"]], **CASES[name])
    log(f"case lost hand-over {name}")
    ws = workspace_for(p)
    bd.debug_handover_fault(True)
    try:
        y_bad = y_to_numpy(call(p, ws))
    finally:
        bd.debug_handover_fault(False)
    assert np.isnan(y_bad).all()
    assert bd.workspace_status(ws) == bd.LORA_EHANDOVER
    assert bd.workspace_status(ws) == bd.LORA_OK          # the query cleared the bits
    ref = lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale)
    assert gates.passes_bf16(y_to_numpy(call(p, ws)), ref)
    assert bd.workspace_status(ws) == bd.LORA_OK


def test_fault_hook_spares_calls_without_adapter_rows():
    """A call whose rows name no adapter waits for nothing, so the hook changes nothing."""
    p = synth.random_problem(73, **CASES["shared_tiles"])
    ws = workspace_for(p)
    base = [-1] * len(p.seg_adapter)
    bd.debug_handover_fault(True)
    try:
        y = y_to_numpy(call(p, ws, seg_adapter=base))
    finally:
        bd.debug_handover_fault(False)
    ref = lora_proj_ref(p.X, p.seg_starts, base, p.W, p.A, p.B, p.scale)
    assert gates.passes_bf16(y, ref)
    assert bd.workspace_status(ws) == bd.LORA_OK
