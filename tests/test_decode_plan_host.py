"""The decode path's launch plan, checked on the host (no GPU).

For a sweep of shapes this replays, from the plan's numbers, the kernel's own assignment of work
to blocks (stream-K over the 64-wide K units of the 128-row weight tiles; each tile's expand units
shared among the blocks whose W range ends in it, or taken whole by a block that covers the tile
and runs past it) and checks that every W unit and every expand unit goes to exactly one block,
that every partial-sum slot fits the workspace the plan lays out, and that the counters fit the
counter area below the error bits."""
from __future__ import annotations

import itertools

import pytest

from rank_adapted_gemm_amd import binding as bd

COUNTER_BYTES = bd.WORKSPACE_COUNTER_BYTES


def pstart(b, U, G):
    return b * U // G


def pblock(u, U, G):
    return ((u + 1) * G - 1) // U


def replay(p):
    """Per W tile: units and expand units each block takes (block -> count), as the kernel does."""
    nst, ntW, GW = p["nst"], p["ntW"], p["GW"]
    nEpt = p["n_used"] * 2 * p["nrs"]
    UW = ntW * nst
    w_units = [0] * UW
    e_units = [[0] * nEpt for _ in range(ntW)]
    slots = [set() for _ in range(ntW)]
    for b in range(GW):
        uw0, uw1 = pstart(b, UW, GW), pstart(b + 1, UW, GW)
        if uw1 <= uw0:
            continue
        for u in range(uw0, uw1):
            w_units[u] += 1
            slots[u // nst].add(b)
        t_last = (uw1 - 1) // nst
        r0 = r1 = 0
        if nEpt > 0:
            e_lo = pblock(t_last * nst, UW, GW)
            bb = pblock((t_last + 1) * nst - 1, UW, GW)
            e_hi = bb if pstart(bb + 1, UW, GW) == (t_last + 1) * nst else bb - 1
            n_end = e_hi - e_lo + 1
            assert e_lo <= b <= e_hi and n_end >= 1
            idx = b - e_lo
            r0, r1 = idx * nEpt // n_end, (idx + 1) * nEpt // n_end
        t = (uw0 + nst - 1) // nst
        u = uw0
        while u < uw1:
            end, et, e0, e1 = uw1, t_last, r0, r1
            if nEpt > 0 and t < t_last:          # a whole tile: its W units, then all its expand units
                end, et, e0, e1 = (t + 1) * nst, t, 0, nEpt
                t += 1
            for e in range(e0, e1):
                e_units[et][e] += 1
            u = end
    return w_units, e_units, slots


def check_plan(M, N, K, rank, n_used, slices=None):
    widths = slices or [N]
    p = bd.decode_plan(M, N, K, rank, n_used, slices)
    assert p is not None, (M, N, K)
    S = len(widths)
    trank = rank * S
    mt = 2 if M <= 32 else 4 if M <= 64 else 5 if M <= 80 else 8
    assert p["MT"] == mt
    assert p["nst"] == (K + 63) // 64 and p["ntW"] == (N + 127) // 128 and p["n_used"] == n_used
    if n_used:
        assert p["nrs"] == (rank + 63) // 64 and p["ntA"] == (trank + 127) // 128
        assert 1 <= p["GA"] <= 32
    else:
        assert p["GA"] == 0
    assert 1 <= p["GW"] <= p["ntW"] * p["nst"] and p["GA"] + p["GW"] <= 256   # all resident at once
    w_units, e_units, slots = replay(p)
    assert w_units == [1] * (p["ntW"] * p["nst"]), "a W unit taken by no block or by two"
    for t in range(p["ntW"]):
        assert e_units[t] == [1] * len(e_units[t]), f"tile {t}: expand units {e_units[t]}"
        assert len(slots[t]) <= p["smaxW"]
    # counters: one per W tile, the A, T and finished-tile counts, below the error bits
    assert (p["ntW"] + 3) * 8 <= COUNTER_BYTES - 8
    frag = 4 * 2 * mt * 64 * 16
    assert p["off_cnt"] == 0 and p["off_pa"] >= COUNTER_BYTES
    assert p["pa_bytes"] == n_used * p["ntA"] * p["GA"] * frag
    assert p["off_pa"] + p["pa_bytes"] <= p["off_pw"] and p["pw_bytes"] == p["ntW"] * p["smaxW"] * frag
    assert p["off_pw"] + p["pw_bytes"] <= p["off_th"]
    assert p["t_bytes"] == n_used * M * trank * 2
    assert p["off_th"] + p["t_bytes"] <= p["off_tl"] and p["off_tl"] + p["t_bytes"] <= p["total"]
    if n_used <= 1:
        assert p["total"] == bd.workspace_bytes(M, N, K, rank if n_used else 16, n_used, "bf16", S)
    return p


SHAPES = [(5120, 5120), (17408, 5120), (5120, 17408), (8, 8), (72, 64), (200, 136), (520, 200), (1000, 520),
          (40960, 64), (257, 72)]


@pytest.mark.parametrize("M", [1, 16, 33, 64, 70, 80, 81, 128])
@pytest.mark.parametrize("n_used", [0, 1, 2, 4])
def test_plan_sweep(M, n_used):
    for (N, K), rank in itertools.product(SHAPES, (16, 48, 256)):
        check_plan(M, N, K, rank, n_used)


@pytest.mark.parametrize("M", [6, 70, 128])
def test_plan_sliced(M):
    for widths, K, rank in (([5120] * 3, 5120, 256), ([17408] * 2, 5120, 256), ([256, 512, 256], 200, 48),
                            ([1024, 512, 512], 1024, 64), ([4096, 1024, 1024], 4096, 256),
                            ([17408, 17408], 512, 64), ([256] * 4, 17408, 512)):
        for n_used in (0, 1, 3):
            check_plan(M, sum(widths), K, rank, n_used, widths)


def test_bench_shapes():
    """The suffix stack's calls fill the GPU: 256 blocks, the A blocks first."""
    for N, K, sl in ((5120, 5120, None), (17408, 5120, None), (5120, 17408, None), (15360, 5120, [5120] * 3),
                     (34816, 5120, [17408] * 2)):
        p = check_plan(70, N, K, 256, 1, sl)
        assert p["GA"] + p["GW"] == 256 and p["GA"] >= 1


def test_plan_off_path():
    assert bd.decode_plan(129, 512, 512, 16, 1) is None
    assert bd.decode_plan(0, 512, 512, 16, 1) is None
    assert bd.decode_plan(64, 512, 100, 16, 1) is None     # K % 8 != 0
