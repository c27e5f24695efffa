"""Pins of the parity gates' own helpers (CPU only)."""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import gates


def _bf16_value(bits):
    return float((np.asarray(bits, dtype=np.uint32) << 16).view(np.float32))


def _nearest_by_fractions(y):
    """bf16 nearest to y by exact rational comparison against every candidate in a window."""
    f = np.float32(y)
    c = int(np.asarray(f).view(np.uint32)) >> 16
    best = None
    for cand in range(c - 2, c + 3):
        v = Fraction(_bf16_value(cand))
        d = abs(v - Fraction(float(y)))
        key = (d, cand % 2)   # ties go to the even bit pattern
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def test_bf16_nearest_matches_exact_rounding():
    g = np.random.Generator(np.random.PCG64(11))
    y = g.standard_normal(400) * np.exp(g.uniform(-8, 8, 400))
    got = gates.bf16_nearest_bits(y)
    want = [_nearest_by_fractions(v) for v in y]
    assert [int(v) for v in got] == want


def test_bf16_nearest_no_double_rounding():
    """Just above the midpoint between bf16 1.0 and its successor, float32 rounds to the midpoint
    itself and a second rounding would pick the even neighbour 1.0; the single rounding is up."""
    y = 1.00390625 + 2.0 ** -40
    assert np.float32(y) == np.float32(1.00390625)
    assert int(gates.bf16_nearest_bits(np.array([y]))[0]) == 0x3F81
    assert int(gates.bf16_nearest_bits(np.array([-y]))[0]) == 0xBF81
    # an exact midpoint goes to the even pattern
    assert int(gates.bf16_nearest_bits(np.array([1.00390625]))[0]) == 0x3F80
    assert int(gates.bf16_nearest_bits(np.array([1.01171875]))[0]) == 0x3F82


def test_explained_by_rounding():
    y_ref = np.array([100.3, 100.3, 100.25 + 1e-9])
    rne = _bf16_value(gates.bf16_nearest_bits(y_ref[:1]))     # 100.5 (bf16 step 0.5 at 100)
    other = rne - 0.5
    y = np.array([rne, other, 100.0])
    ok = gates.explained_by_rounding(y, y_ref, rms_ref=1.0)
    # the correct rounding passes; the wrong neighbour far from a tie fails; at a near-tie either
    # neighbour passes
    assert ok.tolist() == [True, False, True]
