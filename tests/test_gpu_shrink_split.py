"""Parity of the prefill shrink split over K, through the C-ABI.

When the grid of 128 x 128 tiles of s X A^T is small and K long, the shrink runs several blocks
per tile, each over its share of K's 64-wide steps; they store fp32 partials and a second kernel
sums them in split order before T is stored.  Each case below splits (the count follows from the
shape alone): 4 splits of 33 steps with the K tail in the last, 8 uneven splits of 65 steps, two
rank tiles of which a rank-16 adapter's second is skipped, a sliced call, and 32 adapters of a few
rows each (32 row tiles where ceil(M/128) is 3: the partials' bound of ceil(M/128) + n_used row
tiles).  Adapters of short interleaved segments and base rows throughout.  Integer inputs: the fp32 store equals the exact
result bit for bit and the bf16 store is its correct rounding.  Gaussian inputs: the G2 bar
against the oracle, and the same bits on a second call."""
from __future__ import annotations

import numpy as np
import pytest

import gates
from gpu_util import log, record, to_device, y_bits, y_to_numpy
from oracle import lora_proj_ref, lora_proj_sliced_ref
from rank_adapted_gemm_amd import binding as bd
from rank_adapted_gemm_amd import synth

pytestmark = pytest.mark.gpu

# shape, adapter ranks (one entry: every adapter at that rank), slice widths, the splits the
# shape gets (min(8, 256 // (ceil(M/128) ceil(trank/128)), ceil(K/64) // 8)), and the adapters
CASES = {
    "k2056": (dict(M=300, N=520, K=2056), [48], None, 4, 3),
    "k4104": (dict(M=300, N=264, K=4104), [32], None, 8, 3),
    "ranked": (dict(M=300, N=520, K=2056), [16, 256, 48], None, 4, 3),
    "sliced": (dict(M=400, N=None, K=1536), [32], [256, 512, 256], 3, 3),
    "many": (dict(M=300, N=264, K=4104), [16], None, 8, 32),
}


def table(seed, M, n_adapters):
    """Segments of 1..60 rows naming one of the adapters or none; with many adapters, segments of
    1..9 rows naming each adapter in turn (every eighth none)."""
    g = np.random.Generator(np.random.PCG64(seed))
    starts, labels = [0], []
    while starts[-1] < M:
        if n_adapters <= 3:
            starts.append(min(M, starts[-1] + int(g.integers(1, 61))))
            labels.append(int(g.integers(-1, n_adapters)))
        else:
            starts.append(min(M, starts[-1] + int(g.integers(1, 10))))
            labels.append(-1 if len(labels) % 8 == 7 else (len(labels) - len(labels) // 8) % n_adapters)
    return starts, labels


def splits(M, K, trank):
    ntn, ntm = -(-trank // 128), -(-M // 128)
    return max(1, min(8, 256 // (ntn * ntm), -(-K // 64) // 8))


def problem(name, seed, integer):
    shape, ranks, slices, _, n_adapters = CASES[name]
    c = dict(shape)
    if slices is not None:
        c["N"] = sum(slices)
    starts, labels = table(seed, c["M"], n_adapters)
    scales = [1.0, 0.5, -2.0] if integer else [0.7, 1.3, -0.4]
    p = synth.random_problem(seed, scale=[scales[a % 3] for a in range(n_adapters)], integer=integer,
                             rank=ranks[0], ranks=ranks if len(ranks) > 1 else ranks * n_adapters,
                             seg_starts=starts, seg_adapter=labels, n_adapters=n_adapters,
                             slices=1 if slices is None else len(slices), **c)
    return p, ranks, slices


def oracle(p, slices):
    if slices is None:
        return lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale)
    return lora_proj_sliced_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale, slices)


def call(p, ranks, slices, dtype):
    import torch
    X, W, A, B = to_device(p)
    if len(ranks) > 1:
        y = bd.lora_proj_ranked(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale, dtype=dtype,
                                slices=slices)
    else:
        y = bd.lora_proj(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale, dtype=dtype,
                         slices=slices)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("name", list(CASES))
def test_split_shrink_exact(name):
    p, ranks, slices = problem(name, 71, integer=True)
    trank = max(ranks) * (1 if slices is None else len(slices))
    assert splits(p.M, p.K, trank) == CASES[name][3] > 1
    assert bd.path(p.M, p.N, p.K, max(ranks)) == "prefill"
    log(f"case split shrink exact {name} M={p.M} N={p.N} K={p.K} ranks={ranks} splits={CASES[name][3]}")
    exact = oracle(p, slices)
    assert np.all(np.abs(exact) < 2 ** 24)
    y32 = y_to_numpy(call(p, ranks, slices, "bf16_f32out"))
    bad = np.argwhere(y32 != exact)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    assert np.array_equal(y_bits(call(p, ranks, slices, "bf16")), gates.bf16_rne_of_f64(exact))


@pytest.mark.parametrize("name", list(CASES))
def test_split_shrink_gaussian(name):
    p, ranks, slices = problem(name, 72, integer=False)
    log(f"case split shrink gaussian {name} M={p.M} N={p.N} K={p.K}")
    ref = oracle(p, slices)
    y = call(p, ranks, slices, "bf16")
    yn = y_to_numpy(y)
    rep = gates.report(yn, ref)
    over = np.abs(yn - ref) > gates.BF16_TOL * rep["rms"]
    log(f"  split/{name} rms={rep['rms']:.4g} G1={rep['g1']:.3e} G2={rep['g2']:.3e} past-G1={int(over.sum())}")
    record(f"split/{name}", rep, int(over.sum()))
    assert rep["nonfinite"] == 0 and rep["g2"] <= gates.BF16_TOL, rep
    if over.any():
        assert gates.explained_by_rounding(yn[over], ref[over], rep["rms"]).all()
    # the partials are summed in a fixed order: a second call gives the same bits
    assert np.array_equal(y_bits(y), y_bits(call(p, ranks, slices, "bf16")))


def test_split_shrink_on_a_dirty_workspace():
    """The ranked case (a rank-16 adapter whose second rank tile is skipped by the shrink and the
    reduction alike) on a workspace whose bytes past the counter area are NaN before the call:
    bitwise the same as on a fresh workspace, so no partial the call did not write is read."""
    import torch
    p, ranks, slices = problem("ranked", 73, integer=False)
    X, W, A, B = to_device(p)
    nbytes = bd.workspace_bytes(p.M, p.N, p.K, max(ranks), len(ranks))
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    ws[:bd.WORKSPACE_COUNTER_BYTES] = 0
    y_dirty = bd.lora_proj_ranked(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale, workspace=ws)
    y_fresh = bd.lora_proj_ranked(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale)
    torch.cuda.synchronize()
    assert np.array_equal(y_bits(y_dirty), y_bits(y_fresh))
    assert not np.isnan(y_to_numpy(y_dirty)).any()
