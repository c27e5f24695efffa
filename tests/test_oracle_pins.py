"""Pins of the fp64 oracle to facts fixed outside its own code.

The oracle is the plain definition of the projection (see oracle/lora_ref.py).
Nothing here re-runs that definition: each pin reaches the answer another way.

  P1  merged weights, brute force — "two 27B models on a single RTX 5090",
      section 3, weights figure: the adapted matrix is W + B.A; section 4,
      request-path figure: running the two thin matrices gives the same result
      as the adapted weights.  Pure-Python loops form W + s B_a A_a and multiply.
  P2  exact rational arithmetic on tiny bf16-valued inputs (fractions.Fraction).
  P3  exact integers: integer inputs make every partial sum exact, so the
      oracle must equal the int64 merged-weight product bit for bit.
  P4  one-hot rows: x = e_i picks column i, y[n] = W[n,i] + s sum_j B[n,j] A[j,i].
  P5  base rows are untouched by the adapter (section 4 request-path figure:
      requests naming the base model use its weights alone, in the same batch).
  P6  linearity in s.   P7  rows are independent (permutation).
  P8  special cases that reduce to a plain product: s = 0, A = 0, B = 0 and an
      all-base table all give X W^T.
  P9  adapters with their own rank and scale in one batch (section 4
      request-path figure: each request runs its own adapter's two thin
      matrices): brute force over W + s_a B_a A_a, exact integers per adapter,
      and a zero-padded smaller rank giving the same rows as the unpadded one.

The last test plants single mistakes in copies of the oracle (a dropped or
sign-flipped term, transposed operands, an off-by-one segment, the wrong
adapter, the scale ignored) and checks that every such mutant fails a pin.
"""
from __future__ import annotations

import fractions
import os

import numpy as np
import pytest

from oracle import lora_proj_ref, lora_proj_sliced_ref, validate_segments
from rank_adapted_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ helpers
def brute_merged(p, rows=None):
    """Pure-Python loops over W + s B_a A_a (the merged adapted weights)."""
    M, K = p.X.shape
    N = p.W.shape[0]
    seg = list(p.seg_starts)
    out = []
    for m in (range(M) if rows is None else rows):
        g = max(i for i in range(len(seg) - 1) if seg[i] <= m)
        while seg[g + 1] <= m:
            g += 1
        a = int(p.seg_adapter[g])
        x = [float(v) for v in p.X[m]]
        y = []
        for n in range(N):
            acc = 0.0
            for k in range(K):
                w = float(p.W[n, k])
                if a >= 0:
                    r = p.A[a].shape[0]
                    w += scale_of(p, a) * sum(float(p.B[a][n, j]) * float(p.A[a][j, k]) for j in range(r))
                acc += x[k] * w
            y.append(acc)
        out.append(y)
    return np.array(out, dtype=np.float64)


def scale_of(p, a):
    """Adapter a's scale: the problem holds one number or one per adapter."""
    return float(p.scale) if np.ndim(p.scale) == 0 else float(p.scale[a])


def call(fn, p, **kw):
    return fn(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale, **kw)


def close(y, ref, rel=1e-12):
    r = max(float(np.sqrt(np.mean(np.square(ref)))), 1e-300)
    return y.shape == ref.shape and float(np.max(np.abs(y - ref))) <= rel * r


# Cases: a rectangular one with two adapters and an empty segment, and a square
# one (N = K = r) where transposed operands still have valid shapes.
def case_rect():
    return synth.random_problem(11, M=7, N=13, K=24, rank=4, seg_starts=[0, 2, 2, 5, 7],
                                seg_adapter=[0, 1, -1, 1], n_adapters=2, scale=0.75)


def case_square():
    return synth.random_problem(12, M=6, N=16, K=16, rank=16, seg_starts=[0, 3, 6],
                                seg_adapter=[-1, 0], n_adapters=1, scale=0.5)


def int_case(scale, square=False):
    if square:
        return synth.random_problem(13, M=24, N=16, K=16, rank=16, seg_starts=[0, 5, 12, 24],
                                    seg_adapter=[0, -1, 0], scale=scale, integer=True)
    return synth.random_problem(14, M=96, N=80, K=256, rank=16,
                                seg_starts=[0, 17, 17, 40, 64, 96], seg_adapter=[-1, 1, 0, -1, 1],
                                n_adapters=2, scale=scale, integer=True)


def exact_int(p):
    """int64 merged-weight product: 2Y = X (2W + 2s_a B_a A_a)^T, exact for integer inputs."""
    X = p.X.astype(np.int64)
    W2 = 2 * p.W.astype(np.int64)
    out = np.empty((p.M, p.N), dtype=np.float64)
    for g in range(len(p.seg_adapter)):
        lo, hi = p.seg_starts[g], p.seg_starts[g + 1]
        a = p.seg_adapter[g]
        if a >= 0:
            s2 = int(round(2 * scale_of(p, a)))
            assert s2 == 2 * scale_of(p, a)
        Wm = W2 if a < 0 else W2 + s2 * (p.B[a].astype(np.int64) @ p.A[a].astype(np.int64))
        out[lo:hi] = (X[lo:hi] @ Wm.T).astype(np.float64) / 2.0
    return out


def onehot_case(scale):
    p = synth.random_problem(15, M=12, N=16, K=16, rank=16, seg_starts=[0, 4, 12],
                             seg_adapter=[-1, 0], scale=scale, integer=True)
    g = np.random.Generator(np.random.PCG64(99))
    cols = g.integers(0, p.K, size=p.M)
    p.X = np.zeros_like(p.X)
    p.X[np.arange(p.M), cols] = 1.0
    return p, cols


def onehot_expected(p, cols):
    out = np.empty((p.M, p.N))
    for m in range(p.M):
        g = int(np.searchsorted(p.seg_starts, m, side="right") - 1)
        a = p.seg_adapter[g]
        i = cols[m]
        for n in range(p.N):
            v = float(p.W[n, i])
            if a >= 0:
                v += p.scale * sum(float(p.B[a][n, j]) * float(p.A[a][j, i]) for j in range(p.A[a].shape[0]))
            out[m, n] = v
    return out


# ------------------------------------------------------------------ the pins
def pin_bruteforce(fn):
    for p in (case_rect(), case_square()):
        if not close(call(fn, p), brute_merged(p)):
            return False
    return True


def pin_rational(fn):
    p = synth.random_problem(16, M=4, N=6, K=16, rank=4, seg_starts=[0, 1, 4],
                             seg_adapter=[-1, 0], scale=0.375)
    F = fractions.Fraction
    s = F(p.scale)
    exact = []
    for m in range(p.M):
        a = -1 if m < 1 else 0
        row = []
        for n in range(p.N):
            v = sum(F(float(p.X[m, k])) * F(float(p.W[n, k])) for k in range(p.K))
            if a >= 0:
                t = [sum(F(float(p.X[m, k])) * F(float(p.A[0][j, k])) for k in range(p.K))
                     for j in range(p.rank)]
                v += s * sum(t[j] * F(float(p.B[0][n, j])) for j in range(p.rank))
            row.append(float(v))
        exact.append(row)
    return close(call(fn, p), np.array(exact), rel=1e-14)


def pin_integer(fn):
    for scale in (1.0, 0.5, 2.0):
        for square in (False, True):
            p = int_case(scale, square)
            if not np.array_equal(call(fn, p), exact_int(p)):
                return False
    return True


def pin_onehot(fn):
    for scale in (0.5, 1.0):
        p, cols = onehot_case(scale)
        if not np.array_equal(call(fn, p), onehot_expected(p, cols)):
            return False
    return True


def pin_base_rows(fn):
    p = int_case(1.0)
    y = call(fn, p)
    base_rows = np.concatenate([np.arange(p.seg_starts[g], p.seg_starts[g + 1])
                                for g in range(len(p.seg_adapter)) if p.seg_adapter[g] < 0])
    q = synth.random_problem(14, M=96, N=80, K=256, rank=16, seg_starts=p.seg_starts,
                             seg_adapter=[-1] * len(p.seg_adapter), n_adapters=2, integer=True)
    y0 = call(fn, q)
    return np.array_equal(y[base_rows], y0[base_rows]) and np.array_equal(y0, p.X.astype(np.float64) @ p.W.T.astype(np.float64))


def pin_linear(fn):
    p = case_rect()
    ys = {}
    for s in (0.0, 1.0, 0.75):
        p.scale = s
        ys[s] = call(fn, p)
    return close(ys[0.75], ys[0.0] + 0.75 * (ys[1.0] - ys[0.0]))


def pin_permutation(fn):
    p = int_case(0.5)
    y = call(fn, p)
    label = np.repeat(np.arange(len(p.seg_adapter)), np.diff(p.seg_starts))
    g = np.random.Generator(np.random.PCG64(3))
    perm = g.permutation(p.M)
    # regroup the permuted rows into one segment per row
    q = synth.random_problem(14, M=96, N=80, K=256, rank=16, seg_starts=np.arange(p.M + 1),
                             seg_adapter=p.seg_adapter[label[perm]], n_adapters=2, scale=0.5, integer=True)
    q.X = p.X[perm]
    return np.array_equal(call(fn, q), y[perm])


def pin_special(fn):
    p = int_case(1.0)
    plain = p.X.astype(np.float64) @ p.W.T.astype(np.float64)
    p.scale = 0.0
    if not np.array_equal(call(fn, p), plain):
        return False
    p.scale = 1.0
    saved = p.A
    p.A = [np.zeros_like(a) for a in saved]
    ok = np.array_equal(call(fn, p), plain)
    p.A = saved
    p.B = [np.zeros_like(b) for b in p.B]
    return ok and np.array_equal(call(fn, p), plain)


def mixed_case(scales, integer=False):
    """Three adapters of ranks 4, 2 and 3 with their own scales, plus base rows."""
    p = synth.random_problem(17, M=40 if integer else 9, N=12, K=20, rank=4,
                             seg_starts=[0, 2, 3, 5, 7, 9] if not integer else [0, 8, 11, 19, 30, 40],
                             seg_adapter=[2, 0, -1, 1, 2], n_adapters=3, scale=list(scales),
                             integer=integer)
    p.A[1], p.B[1] = p.A[1][:2].copy(), p.B[1][:, :2].copy()
    p.A[2], p.B[2] = p.A[2][:3].copy(), p.B[2][:, :3].copy()
    return p


def pin_per_adapter(fn):
    p = mixed_case([0.75, -1.5, 0.25])
    if not close(call(fn, p), brute_merged(p)):
        return False
    for scales in ([1.0, 0.5, 2.0], [0.0, -1.0, 1.5]):
        q = mixed_case(scales, integer=True)
        if not np.array_equal(call(fn, q), exact_int(q)):
            return False
    # padding adapter 1 (rank 2) with zero rows of A and zero columns of B to rank 4
    # leaves every partial sum exact for integer inputs, so the rows agree bit for bit
    y = call(fn, q)
    q.A[1] = np.concatenate([q.A[1], np.zeros((2, q.K), np.float32)])
    q.B[1] = np.concatenate([q.B[1], np.zeros((q.N, 2), np.float32)], axis=1)
    return np.array_equal(call(fn, q), y)


PINS = dict(bruteforce=pin_bruteforce, rational=pin_rational, integer=pin_integer,
            onehot=pin_onehot, base_rows=pin_base_rows, linear=pin_linear,
            permutation=pin_permutation, special=pin_special, per_adapter=pin_per_adapter)


def failed_pins(fn):
    bad = []
    for name, pin in PINS.items():
        try:
            ok = pin(fn)
        except Exception:  # a mutant that crashes fails the pin
            ok = False
        if not ok:
            bad.append(name)
    return bad


@pytest.mark.parametrize("name", list(PINS))
def test_oracle_pin(name):
    assert PINS[name](lora_proj_ref), name


# ------------------------------------------------------------------ mutants
def _mutant(kind):
    def fn(X, seg_starts, seg_adapter, W, A, B, scale, rows=None):
        X = np.asarray(X)
        M = X.shape[0]
        s = np.asarray(seg_starts, dtype=np.int64).copy()
        a = np.asarray(seg_adapter, dtype=np.int64)
        if kind == "segment_off_by_one":
            s[1:-1] = np.minimum(s[1:-1] + 1, M)
        W64 = np.asarray(W, dtype=np.float64)
        scales = [float(scale)] * len(A) if np.ndim(scale) == 0 else [float(v) for v in scale]
        Y = np.empty((M, W64.shape[0]))
        for g in range(len(a)):
            x = X[s[g]:s[g + 1]].astype(np.float64)
            base = x @ (W64 if kind == "W_untransposed" else W64.T)
            ad = int(a[g])
            if kind == "adapter_on_base_rows" and ad < 0:
                ad = 0
            if kind == "wrong_adapter" and ad >= 0:
                ad = (ad + 1) % len(A)
            if ad < 0 or kind == "adapter_dropped":
                Y[s[g]:s[g + 1]] = base
                continue
            A64 = np.asarray(A[ad], dtype=np.float64)
            B64 = np.asarray(B[ad], dtype=np.float64)
            t = x @ (A64 if kind == "A_untransposed" else A64.T)
            d = t @ (B64 if kind == "B_untransposed" else B64.T)
            sc = scales[ad]
            sc = {"scale_ignored": 1.0, "scale_squared": sc * sc, "first_scale_for_all": scales[0],
                  "scale_by_segment": scales[g % len(scales)]}.get(kind, sc)
            Y[s[g]:s[g + 1]] = base - sc * d if kind == "sign_flipped" else base + sc * d
        return Y
    return fn


MUTANTS = ["adapter_dropped", "sign_flipped", "scale_ignored", "scale_squared", "A_untransposed",
           "B_untransposed", "W_untransposed", "segment_off_by_one", "adapter_on_base_rows",
           "wrong_adapter", "first_scale_for_all", "scale_by_segment"]


def test_unmutated_copy_passes_every_pin():
    assert failed_pins(_mutant("none")) == []


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_fails_a_pin(kind):
    assert failed_pins(_mutant(kind)), f"mutant {kind} passed every pin"


# ------------------------------------------------------------------ table checks
def test_segment_table_rules():
    validate_segments([0, 3, 3, 8], [0, -1, 0], 8, 1)          # empty segment is fine
    validate_segments([0], [], 0, 0)                          # M = 0, no segments
    for starts, adapters, M in (([1, 8], [0], 8), ([0, 5], [0], 8), ([0, 6, 4, 8], [0, 0, 0], 8),
                                ([0, 8], [1], 8), ([0, 8], [-2], 8), ([0], [], 8)):
        with pytest.raises(ValueError):
            validate_segments(starts, adapters, M, 1)


def test_empty_batch_and_sampled_rows():
    p = case_rect()
    full = call(lora_proj_ref, p)
    rows = np.array([6, 0, 3])
    assert close(call(lora_proj_ref, p, rows=rows), full[rows], rel=1e-13)
    q = synth.random_problem(1, M=0, N=5, K=8, rank=4, seg_starts=[0], seg_adapter=[])
    assert call(lora_proj_ref, q).shape == (0, 5)


# ------------------------------------------------------------------ golden files
def _read_kv(path):
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(None, 1)
                out[k] = v
    return out


def test_page_counts_fit_the_shape_model():
    """Printed counts (section 3 weights figure; section 4 memory figure) agree with one another
    and bound the seven-projection stand-in used by the workloads."""
    c = _read_kv(os.path.join(GOLDEN, "page_counts.txt"))
    base, adapter, rank = int(c["base_parameters"]), int(c["adapter_parameters"]), int(c["adapter_rank"])
    assert adapter % rank == 0
    assert round((base + adapter) / 1e9, 1) == float(c["one_copy_plus_adapter_billion"])
    assert round(2 * base / 1e9, 1) == float(c["two_copies_billion"])
    assert round(adapter * 2 / 2 ** 30, 1) == float(c["adapter_bf16_gib"])
    layers = int(c["adapted_last"]) - int(c["adapted_first"]) + 1
    assert layers == synth.N_ADAPTED_LAYERS and int(c["total_layers"]) == 64
    assert int(c["hidden_width"]) == 5120 == synth.PROJECTIONS[0][1]
    stand_in = rank * layers * sum(k + n for _, k, n in synth.PROJECTIONS)
    assert stand_in == 666_894_336 and 0.9 < stand_in / adapter < 1.0


def test_tiny_oracle_matches_stored_values():
    """tests/golden/tiny_oracle.txt is written by tests/golden/make_golden.py (oracle only)."""
    c = _read_kv(os.path.join(GOLDEN, "tiny_oracle.txt"))
    p = synth.tiny()
    y = call(lora_proj_ref, p)
    for key, val in c.items():
        if key.startswith("y["):
            m, n = (int(v) for v in key[2:-1].split(","))
            assert abs(y[m, n] - float(val)) <= 1e-12 * abs(float(val)) + 1e-15
    assert abs(np.sqrt(np.mean(y[:32] ** 2)) - float(c["rms_base_rows"])) < 1e-12
    assert abs(np.sqrt(np.mean(y[32:] ** 2)) - float(c["rms_adapter_rows"])) < 1e-12


# ------------------------------------------------------------------ sliced calls
# Several projections of the same rows stored as one matrix (section 4 request-path figure: every
# changed matrix of a group runs the base product plus its own two thin matrices).  The sliced oracle
# is pinned by brute force over each slice's merged weights W_s + s_a B_{a,s} A_{a,s}, exact integers,
# and its reduction to the plain oracle for one slice.
def sliced_case(widths, rank, integer=False, scale=0.75, seed=41):
    N = sum(widths)
    p = synth.random_problem(seed, M=9 if not integer else 48, N=N, K=12 if not integer else 96,
                             rank=rank * len(widths), seg_starts=[0, 2, 5, 9] if not integer else [0, 7, 30, 48],
                             seg_adapter=[1, -1, 0], n_adapters=2, scale=scale, integer=integer)
    # B_a is N x r: keep the first r columns of the drawn N x (S r) matrix
    p.B = [b[:, :rank].copy() for b in p.B]
    return p


def brute_sliced(p, widths):
    """Pure-Python loops over each slice's merged weights W_s + s_a B_{a,s} A_{a,s}."""
    M, K = p.X.shape
    S = len(widths)
    ends = np.cumsum(widths)
    out = np.zeros((M, p.W.shape[0]))
    for m in range(M):
        g = int(np.searchsorted(p.seg_starts, m, side="right") - 1)
        a = int(p.seg_adapter[g])
        for n in range(p.W.shape[0]):
            s = int(np.searchsorted(ends, n, side="right"))
            acc = 0.0
            for k in range(K):
                w = float(p.W[n, k])
                if a >= 0:
                    r = p.A[a].shape[0] // S
                    w += scale_of(p, a) * sum(float(p.B[a][n, j]) * float(p.A[a][s * r + j, k]) for j in range(r))
                acc += float(p.X[m, k]) * w
            out[m, n] = acc
    return out


def call_sliced(fn, p, widths, **kw):
    return fn(p.X, p.seg_starts, p.seg_adapter, p.W, p.A, p.B, p.scale, widths, **kw)


def exact_int_sliced(p, widths):
    """int64 merged product per slice, exact for integer inputs (2Y, halved at the end)."""
    S = len(widths)
    X = p.X.astype(np.int64)
    out = np.empty((p.M, p.W.shape[0]))
    c0 = 0
    for s, w in enumerate(widths):
        W2 = 2 * p.W[c0:c0 + w].astype(np.int64)
        for g in range(len(p.seg_adapter)):
            lo, hi, a = p.seg_starts[g], p.seg_starts[g + 1], p.seg_adapter[g]
            Wm = W2
            if a >= 0:
                r = p.A[a].shape[0] // S
                s2 = int(round(2 * scale_of(p, a)))
                Wm = W2 + s2 * (p.B[a][c0:c0 + w].astype(np.int64) @ p.A[a][s * r:(s + 1) * r].astype(np.int64))
            out[lo:hi, c0:c0 + w] = (X[lo:hi] @ Wm.T).astype(np.float64) / 2.0
        c0 += w
    return out


def pin_sliced_bruteforce(fn):
    for widths, rank in (([4, 8, 4], 2), ([6, 6], 3)):
        p = sliced_case(widths, rank)
        if not close(call_sliced(fn, p, widths), brute_sliced(p, widths)):
            return False
    return True


def pin_sliced_integer(fn):
    for scale in (1.0, 0.5):
        widths = [32, 16, 32]
        p = sliced_case(widths, 8, integer=True, scale=scale)
        if not np.array_equal(call_sliced(fn, p, widths), exact_int_sliced(p, widths)):
            return False
    return True


def pin_sliced_one_slice(fn):
    """One slice is the plain projection, bit for bit."""
    p = case_rect()
    return np.array_equal(call_sliced(fn, p, [p.W.shape[0]]), call(lora_proj_ref, p))


PINS_SLICED = dict(sliced_bruteforce=pin_sliced_bruteforce, sliced_integer=pin_sliced_integer,
                   sliced_one_slice=pin_sliced_one_slice)


@pytest.mark.parametrize("name", list(PINS_SLICED))
def test_sliced_oracle_pin(name):
    assert PINS_SLICED[name](lora_proj_sliced_ref), name


def _sliced_mutant(kind):
    def fn(X, seg_starts, seg_adapter, W, A, B, scale, slice_n, rows=None):
        widths = [int(v) for v in slice_n]
        S = len(widths)
        outs, c0 = [], 0
        for s, w in enumerate(widths):
            As, Bs = [], []
            for a in range(len(A)):
                r = np.asarray(A[a]).shape[0] // S
                sa = 0 if kind == "first_slice_A_everywhere" else (S - 1 - s if kind == "slices_reversed" else s)
                As.append(np.asarray(A[a])[sa * r:(sa + 1) * r])
                b0 = 0 if kind == "B_not_offset" else c0
                Bs.append(np.asarray(B[a])[b0:b0 + w])
            Ws = np.asarray(W)[c0:c0 + w]
            if kind == "W_slice_shifted" and s > 0:
                Ws = np.asarray(W)[c0 - 1:c0 - 1 + w]
            outs.append(lora_proj_ref(X, seg_starts, seg_adapter, Ws, As, Bs, scale, rows=rows))
            c0 += w
        return np.concatenate(outs, axis=1)
    return fn


SLICED_MUTANTS = ["first_slice_A_everywhere", "slices_reversed", "B_not_offset", "W_slice_shifted"]


def test_unmutated_sliced_copy_passes_every_pin():
    f = _sliced_mutant("none")
    assert all(pin(f) for pin in PINS_SLICED.values())


@pytest.mark.parametrize("kind", SLICED_MUTANTS)
def test_planted_sliced_mistake_fails_a_pin(kind):
    f = _sliced_mutant(kind)
    bad = []
    for name, pin in PINS_SLICED.items():
        try:
            ok = pin(f)
        except Exception:
            ok = False
        if not ok:
            bad.append(name)
    assert bad, f"sliced mutant {kind} passed every pin"


# ------------------------------------------------------------------ 4-bit base weights
# "two 27B models on a single RTX 5090", section 4 memory figure: a 4-bit copy of the base weights
# beside the bf16 adapter.  dequantize_q4 is pinned by an element-wise pure-Python decoder written
# from the format description, an exact round trip through hand-packed codes, and a one-code closed
# form that fixes the nibble order.
import struct

from oracle import dequantize_q4, lora_proj_q4_ref


def decode_q4_loops(packed, params, K):
    """Element by element: code from its nibble, scale and zero from the group's word."""
    N = packed.shape[0]
    out = np.zeros((N, K))
    for n in range(N):
        for k in range(K):
            byte = int(packed[n, k // 2])
            code = (byte & 0xF) if k % 2 == 0 else (byte >> 4)
            word = int(params[k // 128, n])
            scale = struct.unpack("<f", struct.pack("<I", (word & 0xFFFF) << 16))[0]
            zero = (word >> 16) & 0xFF
            out[n, k] = scale * (code - zero)
    return out


def pack_by_hand(codes, scales_bf16_bits, zeros):
    """Pack codes (N x K) and per-(row, group) params with explicit loops."""
    N, K = codes.shape
    packed = np.zeros((N, K // 2), dtype=np.uint8)
    for n in range(N):
        for j in range(K // 2):
            packed[n, j] = int(codes[n, 2 * j]) | (int(codes[n, 2 * j + 1]) << 4)
    params = np.zeros((K // 128, N), dtype=np.uint32)
    for n in range(N):
        for g in range(K // 128):
            params[g, n] = int(scales_bf16_bits[n, g]) | (int(zeros[n, g]) << 16)
    return packed, params


def grid_case(seed=71, N=6, K=256):
    """Codes, power-of-two scales and zeros drawn at random: every weight s (q - z) is exact."""
    g = np.random.Generator(np.random.PCG64(seed))
    codes = g.integers(0, 16, size=(N, K))
    exps = g.integers(-6, 0, size=(N, K // 128))
    scales = np.ldexp(1.0, exps).astype(np.float32)
    zeros = g.integers(0, 16, size=(N, K // 128))
    packed, params = pack_by_hand(codes, synth.f32_to_bf16_bits(scales), zeros)
    W = np.zeros((N, K))
    for n in range(N):
        for k in range(K):
            W[n, k] = float(scales[n, k // 128]) * (int(codes[n, k]) - int(zeros[n, k // 128]))
    return packed, params, W


def pin_q4_loops(fn):
    W = synth.normal_f32(72, (5, 384), 0.1)
    packed, params, *_ = synth.quantize_q4(W)
    return np.array_equal(fn(packed, params, 384), decode_q4_loops(packed, params, 384))


def pin_q4_grid(fn):
    packed, params, W = grid_case()
    return np.array_equal(fn(packed, params, 256), W)


def pin_q4_one_code(fn):
    """All codes equal their zero point except code k = 1 of row 2 (the high nibble of byte 0)."""
    N, K = 4, 256
    codes = np.full((N, K), 5)
    codes[2, 1] = 7
    zeros = np.full((N, K // 128), 5)
    scales = np.full((N, K // 128), 0.25, dtype=np.float32)
    packed, params = pack_by_hand(codes, synth.f32_to_bf16_bits(scales), zeros)
    W = fn(packed, params, K)
    expect = np.zeros((N, K))
    expect[2, 1] = 0.5
    return np.array_equal(W, expect)


PINS_Q4 = dict(q4_loops=pin_q4_loops, q4_grid=pin_q4_grid, q4_one_code=pin_q4_one_code)


@pytest.mark.parametrize("name", list(PINS_Q4))
def test_q4_dequant_pin(name):
    assert PINS_Q4[name](dequantize_q4), name


def test_q4_projection_is_the_plain_projection_of_the_exact_weights():
    packed, params, W = grid_case(N=8, K=256)
    p = synth.random_problem(73, M=5, N=8, K=256, rank=4, seg_starts=[0, 2, 5], seg_adapter=[0, -1], integer=True)
    y = lora_proj_q4_ref(p.X, p.seg_starts, p.seg_adapter, packed, params, p.A, p.B, 0.5)
    assert np.array_equal(y, lora_proj_ref(p.X, p.seg_starts, p.seg_adapter, W, p.A, p.B, 0.5))
    ys = lora_proj_q4_ref(p.X, p.seg_starts, p.seg_adapter, packed, params, [a * 0 for a in p.A], p.B, 0.5)
    assert np.array_equal(ys, p.X.astype(np.float64) @ W.T)


def _q4_mutant(kind):
    def fn(packed, params, K):
        packed = np.asarray(packed, dtype=np.uint8)
        params = np.asarray(params, dtype=np.uint32)
        N = packed.shape[0]
        q = np.empty((N, K))
        lo, hi = packed & 0xF, packed >> 4
        q[:, 0::2], q[:, 1::2] = (hi, lo) if kind == "nibbles_swapped" else (lo, hi)
        scale = ((params & 0xFFFF).astype(np.uint32) << 16).view(np.float32).astype(np.float64).T
        zero = ((params >> 16) & 0xFF).astype(np.float64).T
        if kind == "zero_ignored":
            zero = zero * 0
        g = np.arange(K) // (64 if kind == "group_of_64" else 128)
        g = np.minimum(g, scale.shape[1] - 1)
        if kind == "scale_of_next_row":
            scale = np.roll(scale, 1, axis=0)
        return scale[:, g] * (q - zero[:, g])
    return fn


@pytest.mark.parametrize("kind", ["nibbles_swapped", "zero_ignored", "group_of_64", "scale_of_next_row"])
def test_planted_q4_mistake_fails_a_pin(kind):
    f = _q4_mutant(kind)
    assert all(pin(_q4_mutant("none")) for pin in PINS_Q4.values())
    bad = []
    for name, pin in PINS_Q4.items():
        try:
            ok = pin(f)
        except Exception:
            ok = False
        if not ok:
            bad.append(name)
    assert bad, f"q4 mutant {kind} passed every pin"
