"""Parity of the HIP path with the fp64 oracle, through the C-ABI.

Bars (per call, over every element compared):
  * bf16 output: G2 — max(|Y - Y_o| - half bf16 ulp of Y_o) <= 2e-2 rms(Y_o); G1 (the literal
    max |Y - Y_o| <= 2e-2 rms(Y_o)) is reported and asserted where it is expected to hold;
  * fp32 test mode: max |Y - Y_o| <= 1e-5 rms(Y_o);
  * bf16 inputs with an fp32 store (diagnostic): max |Y - Y_o| <= 3e-5 rms(Y_o);
  * integer-valued inputs: every partial sum is an exact integer below 2^24, so the fp32 store
    must equal the exact result bit for bit and the bf16 store must be its correct rounding.
"""
from __future__ import annotations

import numpy as np
import pytest

import gates
from gpu_util import log, record, run, to_device, y_bits, y_to_numpy
from oracle import lora_proj_q4_ref, lora_proj_ref, lora_proj_sliced_ref
from rank_adapted_gemm_amd import binding as bd
from rank_adapted_gemm_amd import synth

pytestmark = pytest.mark.gpu

F32OUT_TOL = 3e-5


def oracle(p, rows=None, scale=None, seg_adapter=None):
    return lora_proj_ref(p.X, p.seg_starts, p.seg_adapter if seg_adapter is None else seg_adapter,
                         p.W, p.A, p.B, p.scale if scale is None else scale, rows=rows)


def check_bf16(p, y_dev, ref, rows=None, literal=True):
    """G2 must hold.  With literal=True G1 must hold too; otherwise every element past the literal
    G1 bound must be the correct bf16 rounding of the oracle value (or lie at a near-tie), so that
    rounding alone explains it."""
    y = y_to_numpy(y_dev) if not isinstance(y_dev, np.ndarray) else y_dev
    if rows is not None:
        y = y[rows]
    rep = gates.report(y, ref)
    over = np.abs(y - ref) > gates.BF16_TOL * rep["rms"]
    log(f"  {p.name} bf16 rms={rep['rms']:.4g} G1={rep['g1']:.3e} G2={rep['g2']:.3e} "
        f"past-G1={int(over.sum())}")
    record(p.name, rep, int(over.sum()))
    assert rep["nonfinite"] == 0
    assert rep["g2"] <= gates.BF16_TOL, rep
    if literal:
        assert rep["g1"] <= gates.BF16_TOL, rep
    elif over.any():
        ok = gates.explained_by_rounding(y[over], ref[over], rep["rms"])
        assert ok.all(), f"{int((~ok).sum())} elements past G1 that rounding does not explain"
    return rep


def check_f32out(p, y_dev, ref, rows=None, tol=F32OUT_TOL):
    y = y_to_numpy(y_dev)
    if rows is not None:
        y = y[rows]
    rep = gates.report(y, ref)
    log(f"  {p.name} f32-out rms={rep['rms']:.4g} err/rms={rep['g1']:.3e}")
    assert rep["nonfinite"] == 0 and rep["g1"] <= tol, rep
    return rep


# ------------------------------------------------------------------ tiny
def test_tiny_fp32_test_mode():
    p = synth.tiny()
    log(f"case tiny f32 path={bd.path(p.M, p.N, p.K, p.rank, 'f32')}")
    y = y_to_numpy(run(p))
    rep = gates.report(y, oracle(p))
    log(f"  tiny f32 err/rms={rep['g1']:.3e}")
    assert rep["nonfinite"] == 0 and rep["g1"] <= gates.F32_TOL, rep


def test_tiny_shapes_bf16():
    p = synth.random_problem(1, M=64, N=512, K=256, rank=16, seg_starts=[0, 32, 64], seg_adapter=[-1, 0],
                             scale=0.5, sigma_w=1 / 16)
    log(f"case tiny-bf16 path={bd.path(p.M, p.N, p.K, p.rank)}")
    ref = oracle(p)
    check_bf16(p, run(p), ref)
    check_f32out(p, run(p, dtype="bf16_f32out"), ref)


# ------------------------------------------------------------------ exact integer cases
INT_CASES = {
    # prefill path: two row tiles with a ragged tail, ragged N (2 x 256 + 8), ragged K and rank,
    # two adapters, a mixed tile holding base rows next to adapter rows of both adapters
    "prefill_ragged": dict(M=300, N=520, K=200, rank=48, seg_starts=[0, 5, 130, 131, 300],
                           seg_adapter=[-1, 0, -1, 1], n_adapters=2),
    # decode path: 64 adapter rows then six one-row base segments
    "decode_suffix": dict(M=70, N=520, K=200, rank=48, seg_starts=[0, 64, 65, 66, 67, 68, 69, 70],
                          seg_adapter=[0, -1, -1, -1, -1, -1, -1], n_adapters=1),
    "single_row": dict(M=1, N=64, K=64, rank=16, seg_starts=[0, 1], seg_adapter=[0], n_adapters=1),
    # odd N takes the element-wise store; one segment over a ragged third row tile
    "odd_n": dict(M=513, N=257, K=72, rank=16, seg_starts=[0, 513], seg_adapter=[0], n_adapters=1),
    "max_rank": dict(M=200, N=96, K=64, rank=512, seg_starts=[0, 100, 200], seg_adapter=[0, -1], n_adapters=1),
}


@pytest.mark.parametrize("name", list(INT_CASES))
@pytest.mark.parametrize("scale", [1.0, 0.5])
def test_integer_exact(name, scale):
    c = INT_CASES[name]
    p = synth.random_problem(7, scale=scale, integer=True, **c)
    p.name = name
    log(f"case int {name} s={scale} path={bd.path(p.M, p.N, p.K, p.rank)}")
    exact = oracle(p)
    assert np.all(np.abs(exact) < 2 ** 24)
    y32 = y_to_numpy(run(p, dtype="bf16_f32out"))
    bad = np.argwhere(y32 != exact)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    yb = y_bits(run(p, dtype="bf16"))
    assert np.array_equal(yb, gates.bf16_rne_of_f64(exact))


@pytest.mark.parametrize("M", [32, 33, 64, 65, 80, 81, 127, 128])
def test_decode_row_heights_exact(M):
    """The decode kernel comes in four activation heights (M up to 32, 64, 80 and 128 rows); each
    side of every boundary, with two adapters and base rows, integer inputs, exact."""
    s = [0, M // 3, M // 3 + 1, M - 2, M]
    p = synth.random_problem(31 + M, M=M, N=392, K=200, rank=48, seg_starts=s, seg_adapter=[0, -1, 1, -1],
                             n_adapters=2, integer=True)
    p.name = f"decode height M={M}"
    assert bd.path(M, p.N, p.K, p.rank) == "decode"
    log(f"case {p.name}")
    exact = oracle(p)
    y32 = y_to_numpy(run(p, dtype="bf16_f32out"))
    bad = np.argwhere(y32 != exact)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    assert np.array_equal(y_bits(run(p, dtype="bf16")), gates.bf16_rne_of_f64(exact))

# ------------------------------------------------------------------ workloads
@pytest.fixture(scope="module")
def layer_inputs():
    cache = {}

    def get(name, layer, K):
        key = (name, layer, K)
        if key not in cache:
            w = synth.WORKLOADS[name]
            cache[key] = synth.layer_input(w["cfg"], layer, w["M"], K)
        return cache[key]
    return get


def workload(layer_inputs, name, proj, layer=0):
    K = synth.projections(name)[proj][1]
    return synth.workload_problem(name, layer=layer, proj=proj, x=layer_inputs(name, layer, K))


@pytest.mark.parametrize("proj", range(7))
def test_suffix_decode_full(layer_inputs, proj):
    """64 adapter rows + 6 base-only decode rows, every row and column checked."""
    p = workload(layer_inputs, "suffix", proj)
    log(f"case suffix proj={proj} path={bd.path(p.M, p.N, p.K, p.rank)}")
    assert bd.path(p.M, p.N, p.K, p.rank) == "decode"
    ref = oracle(p)
    check_bf16(p, run(p), ref)


@pytest.mark.parametrize("proj", range(7))
def test_mixed_batch(layer_inputs, proj):
    """6 base-only decode rows around a 2,048-row adapter chunk: every row and column checked."""
    p = workload(layer_inputs, "mixed", proj)
    log(f"case mixed proj={proj} path={bd.path(p.M, p.N, p.K, p.rank)}")
    ref = oracle(p)
    check_bf16(p, run(p), ref, literal=False)
    check_f32out(p, run(p, dtype="bf16_f32out"), ref)


@pytest.mark.parametrize("proj", range(7))
def test_prefill16k_sampled(layer_inputs, proj):
    """The 16,384-row adapted prefill at full size, in the launch configuration the benchmark times."""
    p = workload(layer_inputs, "prefill16k", proj)
    log(f"case prefill16k proj={proj} path={bd.path(p.M, p.N, p.K, p.rank)}")
    assert bd.path(p.M, p.N, p.K, p.rank) == "prefill"
    rows = synth.sample_rows(p.M, p.seg_starts, 256, seed=100 + proj)
    ref = oracle(p, rows=rows)
    check_bf16(p, run(p), ref, rows=rows, literal=False)


@pytest.mark.parametrize("proj", [0, 4, 6])
def test_stack32k_layer_sampled(layer_inputs, proj):
    p = workload(layer_inputs, "stack32k", proj)
    log(f"case stack32k proj={proj}")
    rows = synth.sample_rows(p.M, p.seg_starts, 192, seed=200 + proj)
    ref = oracle(p, rows=rows)
    check_bf16(p, run(p), ref, rows=rows, literal=False)


# ------------------------------------------------------------------ the 9B backbone's stand-in shapes
@pytest.mark.parametrize("proj", range(7))
def test_9b_suffix_decode_full(layer_inputs, proj):
    p = workload(layer_inputs, "suffix_9b", proj)
    log(f"case suffix_9b proj={proj} N={p.N} K={p.K} path={bd.path(p.M, p.N, p.K, p.rank)}")
    check_bf16(p, run(p), oracle(p))


@pytest.mark.parametrize("proj", range(7))
def test_9b_prefill16k_sampled(layer_inputs, proj):
    p = workload(layer_inputs, "prefill16k_9b", proj)
    log(f"case prefill16k_9b proj={proj} N={p.N} K={p.K}")
    rows = synth.sample_rows(p.M, p.seg_starts, 256, seed=300 + proj)
    check_bf16(p, run(p), oracle(p, rows=rows), rows=rows, literal=False)


@pytest.mark.parametrize("name", ["suffix_9b", "prefill16k_9b"])
def test_9b_qkv_sliced(layer_inputs, name):
    """q, k and v of a 9B layer as one sliced call (slices 4096, 1024, 1024) against the plain
    oracle of each projection: the columns of slice s equal projection s's own result."""
    import torch
    ps = [workload(layer_inputs, name, j) for j in range(3)]
    widths = [p.N for p in ps]
    cat = lambda arrs: np.ascontiguousarray(np.concatenate(arrs, axis=0))
    X, _, _, _ = to_device(ps[0])
    dev = lambda bits: torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    W = dev(cat([p.W_bits for p in ps]))
    A = dev(cat([p.A_bits[0] for p in ps]))
    B = dev(cat([p.B_bits[0] for p in ps]))
    p0 = ps[0]
    log(f"case {name} qkv sliced widths={widths}")
    y = bd.lora_proj(X, list(p0.seg_starts), list(p0.seg_adapter), W, [A], [B], p0.scale, slices=widths)
    torch.cuda.synchronize()
    rows = None if p0.M <= 128 else synth.sample_rows(p0.M, p0.seg_starts, 128, seed=400)
    yv = y_to_numpy(y)
    c0 = 0
    for p, w in zip(ps, widths):
        ref = oracle(p, rows=rows)
        got = yv[:, c0:c0 + w] if rows is None else yv[rows, c0:c0 + w]
        rep = gates.report(got, ref)
        log(f"  slice {p.name}: G2={rep['g2']:.3e}")
        assert rep["nonfinite"] == 0 and rep["g2"] <= gates.BF16_TOL, rep
        c0 += w


# ------------------------------------------------------------------ invariants
@pytest.mark.parametrize("name", ["mixed", "suffix"])
def test_base_rows_bitwise_unchanged_by_adapter(layer_inputs, name):
    """Rows of base-only requests come out identical whether or not other rows use the adapter."""
    p = workload(layer_inputs, name, 0)
    log(f"case base-row invariance {name}")
    dev = to_device(p)
    y_mixed = y_bits(run(p, dev_inputs=dev))
    y_plain = y_bits(run(p, dev_inputs=dev, seg_adapter=[-1] * len(p.seg_adapter)))
    base = np.concatenate([np.arange(p.seg_starts[g], p.seg_starts[g + 1])
                           for g in range(len(p.seg_adapter)) if p.seg_adapter[g] < 0])
    a = synth.bf16_bits_to_f32(y_mixed[base])
    b = synth.bf16_bits_to_f32(y_plain[base])
    assert np.array_equal(a, b)          # +0 and -0 compare equal
    adapter_rows = np.setdiff1d(np.arange(p.M), base)
    assert not np.array_equal(y_mixed[adapter_rows], y_plain[adapter_rows])


def test_bitwise_deterministic(layer_inputs):
    p = workload(layer_inputs, "mixed", 6)
    log("case determinism mixed/down")
    dev = to_device(p)
    first = y_bits(run(p, dev_inputs=dev))
    for _ in range(2):
        assert np.array_equal(first, y_bits(run(p, dev_inputs=dev)))


# ------------------------------------------------------------------ edge cases
def test_edge_tables():
    base = dict(M=1000, N=264, K=128, rank=32, n_adapters=3)
    g = np.random.Generator(np.random.PCG64(5))
    cuts = np.sort(g.choice(np.arange(1, 1000), 199, replace=False))
    starts = np.concatenate([[0], cuts, [1000]])
    adapters = g.integers(-1, 3, size=200)
    cases = {
        "many_segments": (starts, adapters),
        "empty_segments": ([0, 0, 10, 10, 500, 1000, 1000], [1, 0, 2, -1, 0, 2]),
        "same_adapter_neighbours": ([0, 100, 200, 300, 1000], [0, 0, 0, -1]),
        "all_base": ([0, 1000], [-1]),
    }
    for name, (s, a) in cases.items():
        p = synth.random_problem(9, seg_starts=s, seg_adapter=a, **base)
        p.name = name
        log(f"case edge {name}")
        check_bf16(p, run(p), oracle(p))


def test_edge_shapes():
    for M, N, K, r in ((1, 5120, 5120, 256), (2, 8, 8, 16), (129, 72, 64, 16), (128, 200, 136, 32),
                       (257, 1000, 520, 256)):
        s = [0, M // 2, M] if M > 1 else [0, 1]
        a = [-1, 0] if M > 1 else [0]
        p = synth.random_problem(21, M=M, N=N, K=K, rank=r, seg_starts=s, seg_adapter=a)
        p.name = f"shape M={M} N={N} K={K} r={r}"
        log(f"case {p.name} path={bd.path(M, N, K, r)}")
        check_bf16(p, run(p), oracle(p))


def test_scale_zero_equals_base():
    p = synth.random_problem(3, M=300, N=256, K=256, rank=32, seg_starts=[0, 300], seg_adapter=[0], scale=0.0)
    dev = to_device(p)
    a = synth.bf16_bits_to_f32(y_bits(run(p, dev_inputs=dev)))
    b = synth.bf16_bits_to_f32(y_bits(run(p, dev_inputs=dev, seg_adapter=[-1])))
    assert np.array_equal(a, b)


def test_shared_workspace_across_paths_and_shapes():
    """One zero-filled workspace serves prefill and decode calls of several shapes in a row.

    The prefill path's scratch starts after the counter area, and every decode call tags the
    counters it uses with its own number, so counts left by earlier calls are never taken for a
    later call's; no call reports a lost hand-over.
    """
    import torch
    cases = [synth.random_problem(31, M=300, N=520, K=256, rank=32, seg_starts=[0, 40, 300], seg_adapter=[-1, 0]),
             synth.random_problem(32, M=70, N=1000, K=520, rank=32, seg_starts=[0, 64, 70], seg_adapter=[0, -1]),
             synth.random_problem(33, M=9, N=136, K=1032, rank=48, seg_starts=[0, 3, 9], seg_adapter=[-1, 0]),
             synth.random_problem(34, M=128, N=520, K=256, rank=32, seg_starts=[0, 128], seg_adapter=[0])]
    need = max(bd.workspace_bytes(p.M, p.N, p.K, p.rank, 1) for p in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for i, p in enumerate(cases):
            p.name = f"shared workspace call {rep}.{i} M={p.M} N={p.N} K={p.K}"
            log(f"case {p.name} path={bd.path(p.M, p.N, p.K, p.rank)}")
            X, W, A, B = to_device(p)
            y = bd.lora_proj(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale, workspace=ws)
            torch.cuda.synchronize()
            check_bf16(p, y, oracle(p))
            assert bd.workspace_status(ws) == bd.LORA_OK


def test_empty_batch():
    import torch
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((32, 64), dtype=torch.bfloat16, device="cuda")
    y = bd.lora_proj(X, [0], [], W, [], [], 1.0)
    assert tuple(y.shape) == (0, 32)


# ------------------------------------------------------------------ per-adapter scales and ranks
PER_ADAPTER_CASES = {
    # prefill: three adapters, one with scale 0, a mixed tile of base and adapter rows
    "prefill": dict(M=300, N=520, K=200, rank=48, seg_starts=[0, 5, 130, 131, 200, 300],
                    seg_adapter=[-1, 0, 2, 1, 0], n_adapters=3, scales=[1.0, 0.0, -0.5]),
    # decode: two adapters over 64 rows, then base rows
    "decode": dict(M=70, N=520, K=200, rank=48, seg_starts=[0, 30, 64, 70],
                   seg_adapter=[1, 0, -1], n_adapters=2, scales=[0.5, -2.0]),
}


def padded_problem(c, true_rank, seed=8):
    """Integer problem whose adapter 1 has rank true_rank, stored zero-padded to c["rank"].

    Returns (device problem with padded A_1, B_1; oracle problem with the unpadded ones).
    """
    c = dict(c)
    scales = c.pop("scales")
    p = synth.random_problem(seed, scale=scales, integer=True, **c)
    for arr in (p.A, p.A_bits):
        arr[1][true_rank:] = 0
    for arr in (p.B, p.B_bits):
        arr[1][:, true_rank:] = 0
    q = synth.random_problem(seed, scale=scales, integer=True, **c)
    q.A = list(p.A)
    q.B = list(p.B)
    q.A[1] = p.A[1][:true_rank]
    q.B[1] = p.B[1][:, :true_rank]
    return p, q


@pytest.mark.parametrize("name", list(PER_ADAPTER_CASES))
def test_per_adapter_scales_and_ranks_exact(name):
    """Each adapter its own scale (one of them 0) and adapter 1 of rank 20 passed zero-padded:
    the fp32 store equals the exact result and the bf16 store is its correct rounding."""
    c = PER_ADAPTER_CASES[name]
    p, q = padded_problem(c, true_rank=20)
    p.name = f"per-adapter {name}"
    log(f"case per-adapter int {name} scales={p.scale} path={bd.path(p.M, p.N, p.K, p.rank)}")
    assert bd.path(p.M, p.N, p.K, p.rank) == name
    exact = lora_proj_ref(q.X, q.seg_starts, q.seg_adapter, q.W, q.A, q.B, q.scale)
    assert np.all(np.abs(exact) < 2 ** 24)
    y32 = y_to_numpy(run(p, dtype="bf16_f32out"))
    bad = np.argwhere(y32 != exact)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    assert np.array_equal(y_bits(run(p, dtype="bf16")), gates.bf16_rne_of_f64(exact))


def interleaved_table(seed, M, n_adapters):
    """Segments of 1..40 rows naming a random adapter or none (neighbours may repeat)."""
    g = np.random.Generator(np.random.PCG64(seed))
    starts, labels = [0], []
    while starts[-1] < M:
        starts.append(min(M, starts[-1] + int(g.integers(1, 41))))
        labels.append(int(g.integers(-1, n_adapters)))
    return starts, labels


@pytest.mark.parametrize("M", [700, 2100])
def test_interleaved_adapters_exact(M):
    """Many short segments of four adapters (and base rows) interleaved through a prefill batch, so
    most row tiles hold several adapters and each adapter's rows are scattered over the batch: the
    adapter-sorted shrink gathers them.  Integer inputs, power-of-two scales: the fp32 store equals
    the exact result and the bf16 store is its correct rounding."""
    starts, labels = interleaved_table(40 + M, M, 4)
    p = synth.random_problem(41, scale=[1.0, 0.5, -2.0, 0.25], integer=True, M=M, N=264, K=136, rank=48,
                             seg_starts=starts, seg_adapter=labels, n_adapters=4)
    p.name = f"interleaved M={M}"
    log(f"case interleaved adapters M={M} segments={len(labels)} path={bd.path(p.M, p.N, p.K, p.rank)}")
    assert bd.path(p.M, p.N, p.K, p.rank) == "prefill"
    exact = lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale)
    assert np.all(np.abs(exact) < 2 ** 24)
    y32 = y_to_numpy(run(p, dtype="bf16_f32out"))
    bad = np.argwhere(y32 != exact)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    assert np.array_equal(y_bits(run(p, dtype="bf16")), gates.bf16_rne_of_f64(exact))


def test_sorted_shrink_edge_plans():
    """Adapter-sorted shrink plans at their edges: adapters 0 and 2 of five are named by no row (no
    shrink tiles), adapter 1 has a single row, adapter 3 exactly 128 rows over three segments (one
    whole virtual tile), adapter 4 129 rows (a one-row second tile).  Integer inputs, exact."""
    starts = [0, 40, 41, 100, 150, 209, 250, 260, 339, 410]
    labels = [-1, 1, 3, 4, 3, -1, 3, 4, -1]
    rows = {a: sum(starts[g + 1] - starts[g] for g in range(len(labels)) if labels[g] == a) for a in range(5)}
    assert rows == {0: 0, 1: 1, 2: 0, 3: 128, 4: 129}, rows
    p = synth.random_problem(43, scale=[1.0, 2.0, 1.0, -0.5, 0.25], integer=True, M=410, N=136, K=72, rank=32,
                             seg_starts=starts, seg_adapter=labels, n_adapters=5)
    p.name = "sorted shrink edges"
    log("case sorted shrink edge plans")
    assert bd.path(p.M, p.N, p.K, p.rank) == "prefill"
    exact = lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale)
    assert np.all(np.abs(exact) < 2 ** 24)
    y32 = y_to_numpy(run(p, dtype="bf16_f32out"))
    bad = np.argwhere(y32 != exact)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"


@pytest.mark.parametrize("name", list(PER_ADAPTER_CASES))
def test_per_adapter_scales_random(name):
    """Gaussian inputs, distinct scales per adapter, bf16 gate against the oracle."""
    c = dict(PER_ADAPTER_CASES[name])
    scales = [0.25, 1.0, -0.75][:c["n_adapters"]]
    c.pop("scales")
    c.update(N=1000, K=520, rank=32)
    p = synth.random_problem(23, scale=scales, **c)
    p.name = f"per-adapter random {name}"
    log(f"case {p.name} path={bd.path(p.M, p.N, p.K, p.rank)}")
    check_bf16(p, run(p), oracle(p))
    # one common scale through the per-adapter entry point equals the single-scale call
    dev = to_device(p)
    same = [0.5] * c["n_adapters"]
    assert np.array_equal(y_bits(run(p, dev_inputs=dev, scale=same)), y_bits(run(p, dev_inputs=dev, scale=0.5)))


# ------------------------------------------------------------------ sliced calls
def sliced_problem(seed, widths, rank, integer=False, **kw):
    """A problem whose A[a] stacks one r x K factor per slice and whose B[a] is N x r."""
    p = synth.random_problem(seed, N=sum(widths), rank=rank * len(widths), integer=integer, **kw)
    p.B = [b[:, :rank].copy() for b in p.B]
    if p.B_bits is not None:
        p.B_bits = [b[:, :rank].copy() for b in p.B_bits]
    return p


def run_sliced(p, widths, dtype=None, scale=None):
    import torch
    X, W, A, B = to_device(p)
    y = bd.lora_proj(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, p.scale if scale is None else scale,
                     dtype=dtype or p.dtype, slices=widths)
    torch.cuda.synchronize()
    return y


SLICED_CASES = {
    # three slices, two adapters with their own scales and base rows; ragged K and rank 48
    "prefill": dict(M=300, K=200, seg_starts=[0, 5, 130, 131, 300], seg_adapter=[-1, 0, -1, 1]),
    "decode": dict(M=70, K=200, seg_starts=[0, 30, 64, 70], seg_adapter=[1, 0, -1]),
}


@pytest.mark.parametrize("name", list(SLICED_CASES))
def test_sliced_integer_exact(name):
    """Slices [256, 512, 256]: fp32 store equal to the exact result, bf16 store its correct rounding."""
    widths = [256, 512, 256]
    p = sliced_problem(51, widths, 48, integer=True, n_adapters=2, scale=[1.0, 0.5], **SLICED_CASES[name])
    log(f"case sliced int {name} widths={widths} path={bd.path(p.M, p.N, p.K, 48)}")
    assert bd.path(p.M, p.N, p.K, 48) == name
    exact = lora_proj_sliced_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale, widths)
    assert np.all(np.abs(exact) < 2 ** 24)
    y32 = y_to_numpy(run_sliced(p, widths, dtype="bf16_f32out"))
    bad = np.argwhere(y32 != exact)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    assert np.array_equal(y_bits(run_sliced(p, widths, dtype="bf16")), gates.bf16_rne_of_f64(exact))


@pytest.mark.parametrize("name", list(SLICED_CASES))
def test_sliced_random(name):
    """Gaussian inputs, slices [1024, 512, 512] at rank 64: bf16 gate against the oracle; the
    fp32 test mode within its bar."""
    widths = [1024, 512, 512]
    p = sliced_problem(52, widths, 64, n_adapters=2, scale=[0.75, 1.0], **dict(SLICED_CASES[name], K=1024))
    p.name = f"sliced random {name}"
    log(f"case {p.name} path={bd.path(p.M, p.N, p.K, 64)}")
    ref = lora_proj_sliced_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale, widths)
    check_bf16(p, run_sliced(p, widths), ref)
    q = sliced_problem(53, widths, 64, n_adapters=2, scale=[0.75, 1.0], dtype="f32", **dict(SLICED_CASES[name], K=256))
    q.name = f"sliced f32 {name}"
    rep = gates.report(y_to_numpy(run_sliced(q, widths)),
                       lora_proj_sliced_ref(q.X, q.seg_starts, q.seg_adapter, q.W, q.A, q.B, q.scale, widths))
    log(f"  {q.name} err/rms={rep['g1']:.3e}")
    assert rep["nonfinite"] == 0 and rep["g1"] <= gates.F32_TOL, rep


def test_one_slice_equals_plain_call():
    """A sliced call with one slice is the per-adapter-scale call, bit for bit, on both paths."""
    for M, s, a in ((300, [0, 40, 300], [-1, 0]), (70, [0, 64, 70], [0, -1])):
        p = synth.random_problem(54, M=M, N=768, K=512, rank=32, seg_starts=s, seg_adapter=a, scale=[0.5])
        dev = to_device(p)
        import torch
        X, W, A, B = dev
        y1 = bd.lora_proj(X, s, a, W, A, B, [0.5], slices=[768])
        y2 = bd.lora_proj(X, s, a, W, A, B, [0.5])
        torch.cuda.synchronize()
        assert np.array_equal(y_bits(y1), y_bits(y2))


# ------------------------------------------------------------------ decode grids with more W tiles than blocks
def test_decode_tiles_inside_one_block_exact():
    """K = 64 gives one unit per W tile, so with 320 tiles most blocks cover whole tiles and run
    past them: those tiles' expand units run right after their W units.  Integer inputs, exact."""
    p = synth.random_problem(61, M=70, N=40960, K=64, rank=32, seg_starts=[0, 20, 64, 70], seg_adapter=[1, 0, -1],
                             n_adapters=2, scale=[1.0, 0.5], integer=True)
    p.name = "decode whole-tile blocks"
    log(f"case {p.name} path={bd.path(p.M, p.N, p.K, p.rank)}")
    assert bd.path(p.M, p.N, p.K, p.rank) == "decode"
    exact = oracle(p)
    y32 = y_to_numpy(run(p, dtype="bf16_f32out"))
    bad = np.argwhere(y32 != exact)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"


def test_decode_wide_sliced():
    """Two 17408-wide slices (272 W tiles, more than the grid's W blocks), Gaussian inputs."""
    widths = [17408, 17408]
    p = sliced_problem(62, widths, 64, M=70, K=512, seg_starts=[0, 64, 70], seg_adapter=[0, -1], scale=[1.0])
    p.name = "decode wide sliced"
    log(f"case {p.name} path={bd.path(p.M, p.N, p.K, 64)}")
    ref = lora_proj_sliced_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale, widths)
    check_bf16(p, run_sliced(p, widths), ref)


# ------------------------------------------------------------------ 4-bit base weights
def q4_grid(seed, N, K):
    """Random codes, zero points and power-of-two scales: every dequantized weight is exact in bf16."""
    g = np.random.Generator(np.random.PCG64(seed))
    codes = g.integers(0, 16, size=(N, K)).astype(np.uint8)
    zeros = g.integers(0, 16, size=(N, K // 128)).astype(np.uint32)
    scales = np.ldexp(1.0, g.integers(-5, 0, size=(N, K // 128))).astype(np.float32)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    params = (synth.f32_to_bf16_bits(scales).astype(np.uint32) | (zeros << 16)).T.copy()
    return packed, params


def run_q4(p, packed, params, dtype="bf16", slices=None):
    import torch
    X, _, A, B = to_device(p)
    Wq = torch.from_numpy(np.ascontiguousarray(packed)).to("cuda")
    Wp = torch.from_numpy(np.ascontiguousarray(params).view(np.int32)).to("cuda")
    y = bd.lora_proj_q4(X, list(p.seg_starts), list(p.seg_adapter), Wq, Wp, A, B, p.scale, dtype=dtype,
                        slices=slices)
    torch.cuda.synchronize()
    return y


Q4_CASES = {
    "prefill": dict(M=300, N=520, K=512, rank=48, seg_starts=[0, 5, 130, 131, 300], seg_adapter=[-1, 0, -1, 1]),
    "decode": dict(M=70, N=520, K=512, rank=48, seg_starts=[0, 30, 64, 70], seg_adapter=[1, 0, -1]),
}


@pytest.mark.parametrize("name", list(Q4_CASES))
def test_q4_integer_exact(name):
    c = Q4_CASES[name]
    p = synth.random_problem(81, n_adapters=2, scale=[1.0, 0.5], integer=True, **c)
    packed, params = q4_grid(82, c["N"], c["K"])
    log(f"case q4 int {name} path={bd.path(p.M, p.N, p.K, p.rank)}")
    exact = lora_proj_q4_ref(p.X, p.seg_starts, p.seg_adapter, packed, params, p.A, p.B, p.scale)
    y32 = y_to_numpy(run_q4(p, packed, params, "bf16_f32out"))
    bad = np.argwhere(y32 != exact)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    assert np.array_equal(y_bits(run_q4(p, packed, params, "bf16")), gates.bf16_rne_of_f64(exact))


@pytest.mark.parametrize("name", list(Q4_CASES))
def test_q4_random(name):
    """Gaussian weights through the stand-in quantizer; the kernels round each weight to bf16."""
    c = dict(Q4_CASES[name], N=1024, K=1024, rank=64)
    p = synth.random_problem(83, n_adapters=2, scale=[0.75, 1.0], **c)
    packed, params, *_ = synth.quantize_q4(p.W)
    p.name = f"q4 random {name}"
    log(f"case {p.name}")
    ref = lora_proj_q4_ref(p.X, p.seg_starts, p.seg_adapter, packed, params, p.A, p.B, p.scale)
    check_bf16(p, run_q4(p, packed, params), ref)


def test_q4_sliced_decode_and_suffix_q():
    widths = [512, 512, 1024]
    p = sliced_problem(84, widths, 64, M=70, K=512, seg_starts=[0, 64, 70], seg_adapter=[0, -1], scale=[1.0])
    packed, params, *_ = synth.quantize_q4(p.W)
    p.name = "q4 sliced decode"
    log(f"case {p.name}")
    ref = lora_proj_q4_ref(p.X, p.seg_starts, p.seg_adapter, packed, params, p.A, p.B, p.scale, slice_n=widths)
    check_bf16(p, run_q4(p, packed, params, slices=widths), ref)
    q = synth.workload_problem("suffix", proj=0)
    packed, params, *_ = synth.quantize_q4(q.W)
    q.name = "q4 suffix q (5120 x 5120)"
    log(f"case {q.name}")
    check_bf16(q, run_q4(q, packed, params), lora_proj_q4_ref(q.X, q.seg_starts, q.seg_adapter, packed, params,
                                                             q.A, q.B, q.scale))


# ------------------------------------------------------------------ negative controls
@pytest.mark.parametrize("arm", ["adapter_off", "scale_doubled", "base_rows_given_adapter", "boundary_off_by_one"])
def test_negative_control_fails_gate(arm):
    """Deliberately wrong calls of the right kernels must fail the bf16 gate against the oracle."""
    p = synth.random_problem(17, M=300, N=520, K=256, rank=32, seg_starts=[0, 40, 300], seg_adapter=[-1, 0])
    ref = oracle(p)
    if arm == "adapter_off":
        y = run(p, seg_adapter=[-1, -1])
    elif arm == "scale_doubled":
        y = run(p, scale=2 * p.scale)
    elif arm == "base_rows_given_adapter":
        y = run(p, seg_adapter=[0, 0])
    else:
        q = synth.random_problem(17, M=300, N=520, K=256, rank=32, seg_starts=[0, 41, 300], seg_adapter=[-1, 0])
        y = run(q)
    assert not gates.passes_bf16(y_to_numpy(y), ref), arm


# ------------------------------------------------------------------ streams
def test_call_on_a_second_stream():
    """The wrapper enqueues on the stream it is given: output and zero-filled workspace are
    allocated on that stream, so the counter area's fill is ordered before the kernel even while
    the current stream is busy, and a freed workspace is only reused by later work on it."""
    import torch
    side = torch.cuda.Stream()
    for M, s, a in ((70, [0, 64, 70], [0, -1]), (300, [0, 40, 300], [-1, 0])):
        p = synth.random_problem(90 + M, M=M, N=1000, K=520, rank=32, seg_starts=s, seg_adapter=a)
        p.name = f"second stream M={M}"
        log(f"case {p.name} path={bd.path(p.M, p.N, p.K, p.rank)}")
        X, W, A, B = to_device(p)
        torch.cuda.synchronize()
        busy = torch.randn((4096, 4096), device="cuda")
        outs = []
        for _ in range(4):
            busy = busy @ busy.t().contiguous() * 1e-3    # keeps the current stream occupied
            outs.append(bd.lora_proj(X, s, a, W, A, B, p.scale, stream=side))   # not the current stream
        torch.cuda.synchronize()
        ref = oracle(p)
        for y in outs:
            check_bf16(p, y, ref)
