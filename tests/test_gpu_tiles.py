"""Parity of each prefill output-tile height (256, 192 and 128 activation rows), through the C-ABI.

The host picks the tile height per shape (lora_proj_tile_rows).  Each case below is a shape that
takes one height, with a ragged last row tile, a K that ends inside a 64-wide stage, a rank that
ends inside one, ragged N, and short segments of three adapters and of base rows interleaved
through the batch.  Integer inputs: the fp32 store must equal the exact result bit for bit and
the bf16 store must be its correct rounding.  Gaussian inputs: the G2 bar against the oracle, and
base-only rows equal to the same call with no adapter rows at all."""
from __future__ import annotations

import numpy as np
import pytest

import gates
from gpu_util import log, record, run, y_bits, y_to_numpy
from oracle import lora_proj_ref
from rank_adapted_gemm_amd import binding as bd
from rank_adapted_gemm_amd import synth

pytestmark = pytest.mark.gpu

# rows, columns, K, and the height the host takes for them
CASES = {
    128: dict(M=300, N=1000, K=136),     # 3 row tiles (128, 128, 44)
    192: dict(M=700, N=11008, K=136),    # 4 row tiles (192 x 3, 124): one wave of 172 tiles
    256: dict(M=700, N=17408, K=136),    # 3 row tiles (256, 256, 188): one wave of 204 tiles
}


def table(seed, M):
    """Segments of 1..60 rows naming one of three adapters or none."""
    g = np.random.Generator(np.random.PCG64(seed))
    starts, labels = [0], []
    while starts[-1] < M:
        starts.append(min(M, starts[-1] + int(g.integers(1, 61))))
        labels.append(int(g.integers(-1, 3)))
    return starts, labels


def problem(tm, seed, integer):
    c = CASES[tm]
    starts, labels = table(seed + tm, c["M"])
    p = synth.random_problem(seed, scale=[1.0, 0.5, -2.0] if integer else [0.7, 1.3, -0.4], integer=integer,
                             rank=48, seg_starts=starts, seg_adapter=labels, n_adapters=3, **c)
    p.name = f"tile{tm}"
    return p


@pytest.mark.parametrize("tm", sorted(CASES))
def test_tile_height_exact(tm):
    p = problem(tm, 91, integer=True)
    assert bd.tile_rows(p.M, p.N, p.K) == tm
    log(f"case tile {tm} exact M={p.M} N={p.N} K={p.K} segments={len(p.seg_adapter)}")
    exact = lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale)
    assert np.all(np.abs(exact) < 2 ** 24)
    y32 = y_to_numpy(run(p, dtype="bf16_f32out"))
    bad = np.argwhere(y32 != exact)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    assert np.array_equal(y_bits(run(p, dtype="bf16")), gates.bf16_rne_of_f64(exact))


@pytest.mark.parametrize("tm", sorted(CASES))
def test_tile_height_gaussian(tm):
    p = problem(tm, 92, integer=False)
    assert bd.tile_rows(p.M, p.N, p.K) == tm
    log(f"case tile {tm} gaussian M={p.M} N={p.N} K={p.K}")
    ref = lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale)
    y = y_to_numpy(run(p))
    rep = gates.report(y, ref)
    over = np.abs(y - ref) > gates.BF16_TOL * rep["rms"]
    log(f"  tile{tm} rms={rep['rms']:.4g} G1={rep['g1']:.3e} G2={rep['g2']:.3e} past-G1={int(over.sum())}")
    record(f"tile{tm}", rep, int(over.sum()))
    assert rep["nonfinite"] == 0 and rep["g2"] <= gates.BF16_TOL, rep
    if over.any():
        assert gates.explained_by_rounding(y[over], ref[over], rep["rms"]).all()
    # base-only rows: bitwise the same as in a call where no row names an adapter
    base = np.repeat(np.array(p.seg_adapter) < 0, np.diff(p.seg_starts))
    y0 = y_to_numpy(run(p, seg_adapter=[-1] * len(p.seg_adapter)))
    assert np.array_equal(y[base], y0[base])


@pytest.mark.parametrize("tm", sorted(CASES))
@pytest.mark.parametrize("K", [64, 72, 128, 200])
def test_tile_height_few_stages(tm, K):
    """One to four 64-wide K stages (the 72 and 200 with a K tail): the loads that a short loop
    issues past its last stage must read zeros and land nowhere that a stage reads.  Integer
    inputs, exact."""
    c = dict(CASES[tm], K=K)
    starts, labels = table(93 + tm + K, c["M"])
    p = synth.random_problem(94, scale=[1.0, 0.5, -2.0], integer=True, rank=48, seg_starts=starts,
                             seg_adapter=labels, n_adapters=3, **c)
    assert bd.tile_rows(p.M, p.N, p.K) == tm
    log(f"case tile {tm} K={K} exact M={p.M} N={p.N}")
    exact = lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale)
    y32 = y_to_numpy(run(p, dtype="bf16_f32out"))
    bad = np.argwhere(y32 != exact)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
