"""A seeded sweep of random calls through the C-ABI, every one checked exactly against the oracle.

Each case draws its own shape and call:
- M from 1 to 900 rows, or 2,000 to 4,200 with N from 3,000 to 4,600, so both the decode and the
  prefill kernels run, and on prefill every output tile height;
- any K that is a multiple of 8 up to 1,344: ragged 64-wide stages, and long enough at small M
  for the shrink to split over K;
- any N up to 1,100, or 2 to 4 slices of multiples of 256 columns;
- 1 to 6 adapters at one rank or each at its own (16 to 512), power-of-two scales of either sign;
- a segment table of random lengths (empty segments included) naming any adapter or none.
Inputs are integers in -2..2, so every partial sum is an integer below 2^24: the fp32 store must
equal the exact result bit for bit and the bf16 store must be its correct rounding.

A second sweep does the same for calls with 4-bit base weights (K a multiple of 128, one rank
for every adapter): random codes and zero points with power-of-two group scales from 2^-5 to
2^-1, so every dequantized weight is exact in bf16 and every partial sum is a multiple of 2^-5
below 2^19, again exact in fp32.  Two more take the first sweep's calls on Gaussian inputs: in
bf16 against the rounding-aware G2 bound (and every element past the literal G1 bound must be
the correct bf16 rounding of the oracle value), and in the fp32 test mode (fp32 inputs and
arithmetic) against the 1e-5 rms bound."""
from __future__ import annotations

import numpy as np
import pytest

import gates
from gpu_util import log, record, to_device, y_bits, y_to_numpy
from oracle import lora_proj_q4_ref, lora_proj_ref, lora_proj_sliced_ref
from rank_adapted_gemm_amd import binding as bd
from rank_adapted_gemm_amd import synth

N_CASES = 96
RANKS = (16, 32, 48, 64, 96, 128, 256, 512)
SCALES = (1.0, 0.5, -2.0, 0.25, -1.0)


def case(i):
    """The i-th call of the sweep: shape, table, ranks, scales and slices (seeded, host only)."""
    g = np.random.Generator(np.random.PCG64(9000 + i))
    kind = g.random()
    large = kind >= 0.85
    if kind < 0.35:
        M = int(g.integers(1, 129))
    else:
        M = int(g.integers(2000, 4201)) if large else int(g.integers(129, 901))
    K = 8 * int(g.integers(1, 169))
    if g.random() < 0.3:
        widths = [256 * int(g.integers(3, 7) if large else g.integers(1, 3)) for _ in range(int(g.integers(2, 5)))]
    else:
        widths = None
    N = sum(widths) if widths else int(g.integers(3000, 4601) if large else g.integers(1, 1101))
    n_ad = int(g.integers(1, 7))
    ranked = g.random() < 0.5
    # every partial sum stays an exact fp32 integer: |x w| sums to at most 4 K, |T| to 4 K |s|,
    # and the expand to 2 r (4 K |s|)
    rmax = max(r for r in RANKS if 4 * K + 2 * r * 8 * K < 2 ** 24)
    pick = lambda: int(g.choice([r for r in RANKS if r <= rmax]))
    ranks = [pick() for _ in range(n_ad)] if ranked else [pick()] * n_ad
    scales = [float(g.choice(SCALES)) for _ in range(n_ad)]
    starts, labels = [0], []
    while starts[-1] < M:
        n = 0 if g.random() < 0.05 else int(g.integers(1, max(2, M // 3 + 1)))
        starts.append(min(M, starts[-1] + n))
        labels.append(int(g.integers(-1, n_ad)))
    return dict(M=M, N=N, K=K, widths=widths, ranks=ranks, ranked=ranked, scales=scales,
                seg_starts=starts, seg_adapter=labels)


def problem(i):
    c = case(i)
    S = len(c["widths"]) if c["widths"] else 1
    p = synth.random_problem(9000 + i, M=c["M"], N=c["N"], K=c["K"], rank=c["ranks"][0], integer=True,
                             ranks=c["ranks"], n_adapters=len(c["ranks"]), slices=S, scale=c["scales"],
                             seg_starts=c["seg_starts"], seg_adapter=c["seg_adapter"])
    return c, p


def exact_of(c, p):
    if c["widths"] is None:
        return lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale)
    return lora_proj_sliced_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale, c["widths"])


def call(c, p, dev, dtype):
    import torch
    X, W, A, B = dev
    if c["ranked"]:
        y = bd.lora_proj_ranked(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, c["scales"], dtype=dtype,
                                slices=c["widths"])
    else:
        y = bd.lora_proj(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, c["scales"], dtype=dtype,
                         slices=c["widths"])
    torch.cuda.synchronize()
    return y


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_call_exact(i):
    c, p = problem(i)
    log(f"case random {i}: M={c['M']} N={c['N']} K={c['K']} slices={c['widths']} ranks={c['ranks']} "
        f"ranked={c['ranked']} segments={len(c['seg_adapter'])} path={bd.path(c['M'], c['N'], c['K'], max(c['ranks']))}")
    exact = exact_of(c, p)
    assert np.all(np.abs(exact) < 2 ** 24)
    dev = to_device(p)
    y32 = y_to_numpy(call(c, p, dev, "bf16_f32out"))
    bad = np.argwhere(y32 != exact)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    assert np.array_equal(y_bits(call(c, p, dev, "bf16")), gates.bf16_rne_of_f64(exact))


def test_random_sweep_covers_its_features():
    """Host only: the sweep's calls are valid and reach what it is meant to reach: both kernel
    paths, every prefill tile height, K tails, split shrinks, slices, mixed ranks, empty segments,
    base-only rows and several adapters in one call."""
    seen = dict(decode=0, prefill=0, tail=0, sliced=0, ranked=0, empty=0, base=0, several=0, split=0)
    heights = set()
    for i in range(N_CASES):
        c = case(i)
        M, N, K, ranks = c["M"], c["N"], c["K"], c["ranks"]
        assert 1 <= M <= 4200 and K % 8 == 0 and 1 <= N <= 6 * 256 * 4
        assert all(16 <= r <= 512 and r % 16 == 0 for r in ranks) and len(ranks) <= bd.MAX_ADAPTERS
        assert 4 * K + 2 * max(ranks) * 8 * K < 2 ** 24
        st, lab = c["seg_starts"], c["seg_adapter"]
        assert st[0] == 0 and st[-1] == M and all(a <= b for a, b in zip(st, st[1:]))
        assert len(lab) == len(st) - 1 and all(-1 <= a < len(ranks) for a in lab)
        path = bd.path(M, N, K, max(ranks))
        seen[path] += 1
        if path == "prefill":
            heights.add(bd.tile_rows(M, N, K))
            trank = max(ranks) * (len(c["widths"]) if c["widths"] else 1)
            ntn, ntm = -(-trank // 128), -(-M // 128)
            seen["split"] += min(8, 256 // (ntn * ntm), -(-K // 64) // 8) > 1
        seen["tail"] += K % 64 != 0
        seen["sliced"] += c["widths"] is not None
        seen["ranked"] += c["ranked"] and len(set(ranks)) > 1
        seen["empty"] += any(a == b for a, b in zip(st, st[1:]))
        seen["base"] += -1 in lab
        seen["several"] += len({a for a in lab if a >= 0}) > 1
    assert all(v >= 2 for v in seen.values()), seen
    assert heights == {128, 192, 256}, heights


N_GAUSS_CASES = 24


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_GAUSS_CASES))
def test_random_call_gaussian(i):
    """The i-th call of the sweep on Gaussian inputs (the workloads' sigmas) and scales of mixed
    sign: G2 against the oracle, and past the literal G1 bound only correct roundings."""
    c = case(i)
    S = len(c["widths"]) if c["widths"] else 1
    scales = [0.7 * v for v in c["scales"]]
    p = synth.random_problem(9900 + i, M=c["M"], N=c["N"], K=c["K"], rank=c["ranks"][0], ranks=c["ranks"],
                             n_adapters=len(c["ranks"]), slices=S, scale=scales, seg_starts=c["seg_starts"],
                             seg_adapter=c["seg_adapter"])
    c = dict(c, scales=scales)
    log(f"case random gaussian {i}: M={c['M']} N={c['N']} K={c['K']} slices={c['widths']} ranks={c['ranks']}")
    ref = exact_of(c, p)
    y = y_to_numpy(call(c, p, to_device(p), "bf16"))
    rep = gates.report(y, ref)
    over = np.abs(y - ref) > gates.BF16_TOL * rep["rms"]
    log(f"  rms={rep['rms']:.4g} G1={rep['g1']:.3e} G2={rep['g2']:.3e} past-G1={int(over.sum())}")
    record(f"random/{i}", rep, int(over.sum()))
    assert rep["nonfinite"] == 0 and rep["g2"] <= gates.BF16_TOL, rep
    if over.any():
        assert gates.explained_by_rounding(y[over], ref[over], rep["rms"]).all()


# ------------------------------------------------------------------ 4-bit base weights
N_Q4_CASES = 40
Q4_SCALES = (0.5, 0.25, -0.5, 0.125, -0.25)


def q4_case(i):
    """The i-th 4-bit call of the sweep (seeded, host only)."""
    g = np.random.Generator(np.random.PCG64(9500 + i))
    kind = g.random()
    large = kind >= 0.85
    if kind < 0.4:
        M = int(g.integers(1, 129))
    else:
        M = int(g.integers(2000, 3001)) if large else int(g.integers(129, 901))
    K = 128 * int(g.integers(1, 10))
    if g.random() < 0.3:
        widths = [256 * int(g.integers(3, 6) if large else g.integers(1, 3)) for _ in range(int(g.integers(2, 5)))]
    else:
        widths = None
    N = sum(widths) if widths else int(g.integers(3000, 4001) if large else g.integers(1, 1101))
    n_ad = int(g.integers(1, 5))
    # base terms |x w| <= 2 * 7.5 sum to at most 15 K, the expand to 8 |s| r K; all multiples of
    # 2^-5, so exact in fp32 below 2^19
    rmax = max(r for r in RANKS if 15 * K + 8 * 0.5 * r * K < 2 ** 19)
    rank = int(g.choice([r for r in RANKS if r <= rmax]))
    scales = [float(g.choice(Q4_SCALES)) for _ in range(n_ad)]
    starts, labels = [0], []
    while starts[-1] < M:
        n = 0 if g.random() < 0.05 else int(g.integers(1, max(2, M // 3 + 1)))
        starts.append(min(M, starts[-1] + n))
        labels.append(int(g.integers(-1, n_ad)))
    return dict(M=M, N=N, K=K, widths=widths, rank=rank, n_ad=n_ad, scales=scales, seg_starts=starts,
                seg_adapter=labels)


def q4_problem(i):
    c = q4_case(i)
    S = len(c["widths"]) if c["widths"] else 1
    p = synth.random_problem(9500 + i, M=c["M"], N=c["N"], K=c["K"], rank=c["rank"], integer=True,
                             ranks=[c["rank"]] * c["n_ad"], n_adapters=c["n_ad"], slices=S, scale=c["scales"],
                             seg_starts=c["seg_starts"], seg_adapter=c["seg_adapter"])
    g = np.random.Generator(np.random.PCG64(9700 + i))
    N, K = c["N"], c["K"]
    codes = g.integers(0, 16, size=(N, K)).astype(np.uint8)
    zeros = g.integers(0, 16, size=(N, K // 128)).astype(np.uint32)
    gscale = np.ldexp(1.0, g.integers(-5, 0, size=(N, K // 128))).astype(np.float32)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    params = (synth.f32_to_bf16_bits(gscale).astype(np.uint32) | (zeros << 16)).T.copy()
    return c, p, packed, params


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_Q4_CASES))
def test_random_q4_call_exact(i):
    import torch
    c, p, packed, params = q4_problem(i)
    log(f"case random q4 {i}: M={c['M']} N={c['N']} K={c['K']} slices={c['widths']} rank={c['rank']} "
        f"adapters={c['n_ad']} segments={len(c['seg_adapter'])} path={bd.path(c['M'], c['N'], c['K'], c['rank'])}")
    exact = lora_proj_q4_ref(p.X, p.seg_starts, p.seg_adapter, packed, params, p.A, p.B, p.scale,
                             slice_n=c["widths"])
    assert np.all(np.abs(exact) * 32 < 2 ** 24)
    X, _, A, B = to_device(p)
    Wq = torch.from_numpy(np.ascontiguousarray(packed)).to("cuda")
    Wp = torch.from_numpy(np.ascontiguousarray(params).view(np.int32)).to("cuda")

    def run(dtype):
        y = bd.lora_proj_q4(X, list(p.seg_starts), list(p.seg_adapter), Wq, Wp, A, B, c["scales"], dtype=dtype,
                            slices=c["widths"])
        torch.cuda.synchronize()
        return y

    y32 = y_to_numpy(run("bf16_f32out"))
    bad = np.argwhere(y32 != exact)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    assert np.array_equal(y_bits(run("bf16")), gates.bf16_rne_of_f64(exact))


def test_random_q4_sweep_covers_its_features():
    """Host only: the 4-bit sweep's calls are valid and reach both paths, several tile heights,
    slices, several adapters, empty segments and base rows."""
    seen = dict(decode=0, prefill=0, sliced=0, empty=0, base=0, several=0)
    heights = set()
    for i in range(N_Q4_CASES):
        c = q4_case(i)
        M, N, K, r = c["M"], c["N"], c["K"], c["rank"]
        assert K % 128 == 0 and 16 <= r <= 512 and r % 16 == 0
        assert 15 * K + 8 * max(abs(v) for v in Q4_SCALES) * r * K < 2 ** 19
        st, lab = c["seg_starts"], c["seg_adapter"]
        assert st[0] == 0 and st[-1] == M and len(lab) == len(st) - 1
        path = bd.path(M, N, K, r)
        seen[path] += 1
        if path == "prefill":
            heights.add(bd.tile_rows(M, N, K))
        seen["sliced"] += c["widths"] is not None
        seen["empty"] += any(a == b for a, b in zip(st, st[1:]))
        seen["base"] += -1 in lab
        seen["several"] += len({a for a in lab if a >= 0}) > 1
    assert all(v >= 2 for v in seen.values()), seen
    assert len(heights) >= 2, heights


# ------------------------------------------------------------------ fp32 test mode
N_F32_CASES = 16


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_F32_CASES))
def test_random_f32_call(i):
    """The i-th call of the first sweep at its own shape and table (M capped at 600, N at 700),
    in fp32 with Gaussian inputs and scales: within 1e-5 rms of the oracle."""
    import torch
    c = case(i)
    M = min(c["M"], 600)
    starts = [min(v, M) for v in c["seg_starts"]]
    widths = None if c["widths"] is None else [256] * min(len(c["widths"]), 2)
    N = sum(widths) if widths else min(c["N"], 700)
    S = len(widths) if widths else 1
    scales = [0.7 * v for v in c["scales"]]
    p = synth.random_problem(9800 + i, M=M, N=N, K=c["K"], rank=c["ranks"][0], dtype="f32", ranks=c["ranks"],
                             n_adapters=len(c["ranks"]), slices=S, scale=scales, seg_starts=starts,
                             seg_adapter=c["seg_adapter"])
    log(f"case random f32 {i}: M={M} N={N} K={c['K']} slices={widths} ranks={c['ranks']} ranked={c['ranked']}")
    ref = (lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale) if widths is None else
           lora_proj_sliced_ref(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale, widths))
    X, W, A, B = to_device(p)
    entry = bd.lora_proj_ranked if c["ranked"] else bd.lora_proj
    y = entry(X, list(p.seg_starts), list(p.seg_adapter), W, A, B, scales, dtype="f32", slices=widths)
    torch.cuda.synchronize()
    assert gates.passes_f32(y_to_numpy(y), ref), gates.report(y_to_numpy(y), ref)
