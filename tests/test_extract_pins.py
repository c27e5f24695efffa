"""Pins of the adapter-extraction oracle (oracle/extract_ref.py) to facts fixed outside its code.

"two 27B models on a single RTX 5090", TL;DR: the adapted weights differ from the base weights by a
merged rank-256 change, which factors back out into an adapter.  The oracle's reading is a truncated
SVD of the change.  Pins, none of which re-runs the oracle's own SVD call:

  E1  planted rank: a change that is exactly a rank-r product comes back exactly (B A = D).
  E2  diagonal change: the singular values are the sorted magnitudes of the diagonal, and B A keeps
      exactly the r largest entries.
  E3  Eckart-Young: the residual's squared norm is the sum of the discarded eigenvalues of D^T D
      (numpy's symmetric eigensolver, a different routine).
  E4  orthogonal invariance: extracting from Q1 D Q2 gives Q1 (B A) Q2.
  E5  the even split: column i of B and row i of A both have norm sqrt(s_i), and s is descending.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import extract_ref


def planted(seed=1, N=40, K=56, r=6, noise=0.0):
    g = np.random.Generator(np.random.PCG64(seed))
    Wb = g.standard_normal((N, K))
    B0, A0 = g.standard_normal((N, r)), g.standard_normal((r, K))
    return Wb + B0 @ A0 + noise * g.standard_normal((N, K)), Wb, B0 @ A0


def rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def pin_planted(fn):
    Wa, Wb, D = planted()
    B, A, s = fn(Wa, Wb, 6)
    return rel(B @ A, D) < 1e-10


def pin_diagonal(fn):
    d = np.array([3.0, -7.0, 0.5, 5.0, -1.0])
    D = np.zeros((7, 5))
    D[np.arange(5), np.arange(5)] = d
    B, A, s = fn(D, np.zeros_like(D), 3)
    keep = np.zeros_like(D)
    for i in (1, 3, 0):                         # |d| = 7, 5, 3
        keep[i, i] = d[i]
    return np.allclose(s, [7.0, 5.0, 3.0], rtol=0, atol=1e-12) and np.allclose(B @ A, keep, rtol=0, atol=1e-12)


def pin_eckart_young(fn):
    Wa, Wb, _ = planted(seed=2, noise=0.05)
    D = Wa - Wb
    B, A, s = fn(Wa, Wb, 6)
    ev = np.sort(np.linalg.eigvalsh(D.T @ D))[::-1]
    resid = np.linalg.norm(D - B @ A) ** 2
    return abs(resid - ev[6:].sum()) < 1e-8 * ev.sum() and np.allclose(s ** 2, ev[:6], rtol=1e-9)


def pin_orthogonal(fn):
    Wa, Wb, _ = planted(seed=3, noise=0.05)
    g = np.random.Generator(np.random.PCG64(4))
    Q1, _ = np.linalg.qr(g.standard_normal((40, 40)))
    Q2, _ = np.linalg.qr(g.standard_normal((56, 56)))
    B, A, _ = fn(Wa, Wb, 6)
    B2, A2, _ = fn(Q1 @ Wa @ Q2, Q1 @ Wb @ Q2, 6)
    return rel(B2 @ A2, Q1 @ (B @ A) @ Q2) < 1e-9


def pin_split(fn):
    Wa, Wb, _ = planted(seed=5, noise=0.05)
    B, A, s = fn(Wa, Wb, 6)
    return (np.all(np.diff(s) <= 0) and np.allclose(np.linalg.norm(B, axis=0), np.sqrt(s), rtol=1e-10)
            and np.allclose(np.linalg.norm(A, axis=1), np.sqrt(s), rtol=1e-10))


PINS = dict(planted=pin_planted, diagonal=pin_diagonal, eckart_young=pin_eckart_young,
            orthogonal=pin_orthogonal, split=pin_split)


@pytest.mark.parametrize("name", list(PINS))
def test_extract_pin(name):
    assert PINS[name](extract_ref), name


def _mutant(kind):
    def fn(Wa, Wb, rank):
        D = np.asarray(Wa, np.float64) - (0 if kind == "base_not_subtracted" else np.asarray(Wb, np.float64))
        U, s, Vt = np.linalg.svd(D, full_matrices=False)
        if kind == "smallest_kept":
            U, s, Vt = U[:, ::-1], s[::-1], Vt[::-1]
        r = rank - 1 if kind == "rank_off_by_one" else rank
        root = np.sqrt(s[:r])
        if kind == "uneven_split":
            return U[:, :r] * s[:r], Vt[:r], s[:r]
        if kind == "factors_transposed":
            return (root[:, None] * Vt[:r]).T, (U[:, :r] * root).T, s[:r]
        return U[:, :r] * root, root[:, None] * Vt[:r], s[:r]
    return fn


MUTANTS = ["base_not_subtracted", "smallest_kept", "rank_off_by_one", "uneven_split", "factors_transposed"]


def test_unmutated_copy_passes():
    assert all(pin(_mutant("none")) for pin in PINS.values())


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_fails_a_pin(kind):
    f = _mutant(kind)
    bad = []
    for name, pin in PINS.items():
        try:
            ok = pin(f)
        except Exception:
            ok = False
        if not ok:
            bad.append(name)
    assert bad, f"mutant {kind} passed every pin"
