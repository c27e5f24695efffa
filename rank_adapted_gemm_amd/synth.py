"""Seeded synthetic workloads for the mixed-adapter LoRA projection.

This module draws inputs and nothing else: Gaussian values, their rounding to
bf16, segment tables and row samples.  It holds none of the projection's
arithmetic, so the GPU path and the fp64 oracle can both take their inputs from
it without sharing any of the computation they are checked on.

Workloads (shapes from "two 27B models on a single RTX 5090", section 3's
weights figure: hidden width 5,120, rank-256 change on the last 24 of 64
layers; section 5: 14,000-16,000-token prompts; section 6's table: prompts up
to 32,013 tokens; the TL;DR: six chats beside a prompt grown by four lines):

  tiny       X 64x256, W 512x256, one adapter of rank 16 (A 16x256, B 512x16),
             fp32, rows 0-31 base-only and 32-63 adapter, s = 0.5, seed 0.
  prefill16k one adapted layer, 16,384 rows, all adapter.
  mixed      one layer, 6 base-only decode rows around a 2,048-row adapter chunk.
  stack32k   24 adapted layers, 32,768 rows, all adapter.
  suffix     24 adapted layers, a 64-row adapter suffix plus 6 base-only decode rows.
  prefill16k_9b, suffix_9b  the same two workloads on stand-in shapes of the 9B
             backbone the pages also adapt (one layer each; see PROJECTIONS_9B).

Each adapted layer has seven projections (K -> N): q, k, v, o 5120 -> 5120;
gate, up 5120 -> 17408; down 17408 -> 5120.

Distributions: N(0, v) is read with v a variance (tiny: W ~ N(0, 1/256) is the
unit-output-variance scale for K = 256).  X ~ N(0, 1); W, A, B ~ N(0, 0.02),
i.e. sigma = sqrt(0.02).

Seeds: tiny draws X, W, A, B in that order from one PCG64(0) stream.  Every
other tensor has its own stream, seed = 1_000_000*cfg + 1_000*layer +
10*proj + tensor, with proj q,k,v,o,gate,up,down = 0..6, the layer's
5,120-wide input = 7, its 17,408-wide input = 8, and tensor X/W/A/B = 0/1/2/3.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

SIGMA_WAB = math.sqrt(0.02)

# (name, K, N) for the seven projections of one adapted layer.
PROJECTIONS = (
    ("q", 5120, 5120),
    ("k", 5120, 5120),
    ("v", 5120, 5120),
    ("o", 5120, 5120),
    ("gate", 5120, 17408),
    ("up", 5120, 17408),
    ("down", 17408, 5120),
)
# Stand-in shapes of the 9B backbone ("Clef-Flash", hidden width 4,096; its
# key/value cache holds 4 heads of 256, so k and v are 1,024 wide).  The pages
# print no MLP width: 12,288 (three times the hidden width) stands in.
PROJECTIONS_9B = (
    ("q", 4096, 4096),
    ("k", 4096, 1024),
    ("v", 4096, 1024),
    ("o", 4096, 4096),
    ("gate", 4096, 12288),
    ("up", 4096, 12288),
    ("down", 12288, 4096),
)
RANK = 256
N_ADAPTED_LAYERS = 24
X_NARROW, X_WIDE = 7, 8          # proj index of the layer inputs of width 5120 / 17408
T_X, T_W, T_A, T_B = 0, 1, 2, 3  # tensor index inside a seed

# cfg number -> workload.  Segment tables: seg_starts has n_seg+1 entries,
# seg_adapter n_seg entries (-1 = base-only, else the adapter index).
WORKLOADS = {
    "tiny": dict(cfg=1, M=64, seg_starts=(0, 32, 64), seg_adapter=(-1, 0), layers=1, scale=0.5),
    "prefill16k": dict(cfg=2, M=16384, seg_starts=(0, 16384), seg_adapter=(0,), layers=1, scale=1.0),
    "mixed": dict(cfg=3, M=2054, seg_starts=(0, 1, 2, 3, 2051, 2052, 2053, 2054),
                  seg_adapter=(-1, -1, -1, 0, -1, -1, -1), layers=1, scale=1.0),
    "stack32k": dict(cfg=4, M=32768, seg_starts=(0, 32768), seg_adapter=(0,),
                     layers=N_ADAPTED_LAYERS, scale=1.0),
    "suffix": dict(cfg=5, M=70, seg_starts=(0, 64, 65, 66, 67, 68, 69, 70),
                   seg_adapter=(0, -1, -1, -1, -1, -1, -1), layers=N_ADAPTED_LAYERS, scale=1.0),
    "prefill16k_9b": dict(cfg=6, M=16384, seg_starts=(0, 16384), seg_adapter=(0,), layers=1, scale=1.0,
                          shapes=PROJECTIONS_9B),
    "suffix_9b": dict(cfg=7, M=70, seg_starts=(0, 64, 65, 66, 67, 68, 69, 70),
                      seg_adapter=(0, -1, -1, -1, -1, -1, -1), layers=1, scale=1.0, shapes=PROJECTIONS_9B),
}


def projections(name: str):
    """(name, K, N) of the seven projections of a workload's layers."""
    return WORKLOADS[name].get("shapes", PROJECTIONS)


def seed_of(cfg: int, layer: int, proj: int, tensor: int) -> int:
    return 1_000_000 * cfg + 1_000 * layer + 10 * proj + tensor


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) and return the bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    if not np.all(np.isfinite(a)):
        raise ValueError("inputs must be finite")
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 value of bf16 bit patterns."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(seed: int, shape, sigma: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    return g.standard_normal(shape, dtype=np.float32) * np.float32(sigma)


def normal_bf16(seed: int, shape, sigma: float):
    """(bits uint16, exact float32 values) of N(0, sigma^2) draws rounded to bf16."""
    bits = f32_to_bf16_bits(normal_f32(seed, shape, sigma))
    return bits, bf16_bits_to_f32(bits)


# ---------------------------------------------------------------- problems
@dataclasses.dataclass
class Problem:
    """One projection call: the inputs of Y = X W^T (+ s (X A_a^T) B_a^T on adapter rows).

    Host arrays.  For bf16 problems *_bits hold the bf16 bit patterns and the
    float arrays hold their exact values; for fp32 problems *_bits are None.
    """
    X: np.ndarray
    W: np.ndarray
    A: list
    B: list
    seg_starts: np.ndarray
    seg_adapter: np.ndarray
    scale: object                    # one float, or a sequence with one per adapter
    dtype: str                       # "bf16" or "f32"
    X_bits: np.ndarray | None = None
    W_bits: np.ndarray | None = None
    A_bits: list | None = None
    B_bits: list | None = None
    name: str = ""

    @property
    def M(self): return self.X.shape[0]

    @property
    def K(self): return self.X.shape[1]

    @property
    def N(self): return self.W.shape[0]

    @property
    def rank(self): return self.A[0].shape[0] if self.A else 0


def tiny() -> Problem:
    """The 64x256 fp32 test-mode case; one PCG64(0) stream in the order X, W, A, B."""
    g = np.random.Generator(np.random.PCG64(0))
    X = g.standard_normal((64, 256), dtype=np.float32)
    W = g.standard_normal((512, 256), dtype=np.float32) * np.float32(1.0 / 16.0)
    A = g.standard_normal((16, 256), dtype=np.float32) * np.float32(0.25)
    B = g.standard_normal((512, 16), dtype=np.float32) * np.float32(0.25)
    w = WORKLOADS["tiny"]
    return Problem(X=X, W=W, A=[A], B=[B],
                   seg_starts=np.array(w["seg_starts"], np.int32),
                   seg_adapter=np.array(w["seg_adapter"], np.int32),
                   scale=w["scale"], dtype="f32", name="tiny")


def layer_input(cfg: int, layer: int, M: int, K: int):
    proj = X_NARROW if K in (5120, 4096) else X_WIDE
    return normal_bf16(seed_of(cfg, layer, proj, T_X), (M, K), 1.0)


def projection_weights(cfg: int, layer: int, proj: int, K: int, N: int, rank: int = RANK):
    Wb, Wf = normal_bf16(seed_of(cfg, layer, proj, T_W), (N, K), SIGMA_WAB)
    Ab, Af = normal_bf16(seed_of(cfg, layer, proj, T_A), (rank, K), SIGMA_WAB)
    Bb, Bf = normal_bf16(seed_of(cfg, layer, proj, T_B), (N, rank), SIGMA_WAB)
    return (Wb, Wf), (Ab, Af), (Bb, Bf)


def workload_problem(name: str, layer: int = 0, proj: int = 0, x=None) -> Problem:
    """One projection of a named bf16 workload, drawn by its seed recipe.

    ``x`` may pass a (bits, values) pair already drawn for this layer's input.
    """
    w = WORKLOADS[name]
    cfg, M = w["cfg"], w["M"]
    pname, K, N = projections(name)[proj]
    if x is None:
        x = layer_input(cfg, layer, M, K)
    (Wb, Wf), (Ab, Af), (Bb, Bf) = projection_weights(cfg, layer, proj, K, N)
    return Problem(X=x[1], W=Wf, A=[Af], B=[Bf],
                   seg_starts=np.array(w["seg_starts"], np.int32),
                   seg_adapter=np.array(w["seg_adapter"], np.int32),
                   scale=w["scale"], dtype="bf16",
                   X_bits=x[0], W_bits=Wb, A_bits=[Ab], B_bits=[Bb],
                   name=f"{name}/L{layer}/{pname}")


def random_problem(seed: int, M: int, N: int, K: int, rank: int, seg_starts, seg_adapter,
                   n_adapters: int = 1, scale=1.0, dtype: str = "bf16",
                   sigma_x: float = 1.0, sigma_w: float = SIGMA_WAB, integer: bool = False,
                   ranks=None, slices: int = 1) -> Problem:
    """A seeded problem of any shape, for parity sweeps and edge cases.

    ``integer`` draws integers in {-2..2} instead of Gaussians (exact in every
    precision the path uses).  ``ranks``: one rank per adapter (then ``rank`` is
    ignored), with A[a] of (slices * ranks[a]) x K (the slices' factors stacked)
    and B[a] of N x ranks[a]; by default every adapter has A of rank x K and B
    of N x rank.
    """
    g = np.random.Generator(np.random.PCG64(seed))

    def draw(shape, sigma):
        if integer:
            return g.integers(-2, 3, size=shape).astype(np.float32)
        return g.standard_normal(shape, dtype=np.float32) * np.float32(sigma)

    X = draw((M, K), sigma_x)
    W = draw((N, K), sigma_w)
    if ranks is None:
        A = [draw((rank, K), sigma_w) for _ in range(n_adapters)]
        B = [draw((N, rank), sigma_w) for _ in range(n_adapters)]
    else:
        if len(ranks) != n_adapters:
            raise ValueError("one rank per adapter")
        A = [draw((slices * r, K), sigma_w) for r in ranks]
        B = [draw((N, r), sigma_w) for r in ranks]
    p = Problem(X=X, W=W, A=A, B=B, seg_starts=np.asarray(seg_starts, np.int32),
                seg_adapter=np.asarray(seg_adapter, np.int32), scale=scale, dtype=dtype,
                name=f"random(seed={seed},M={M},N={N},K={K},r={rank if ranks is None else list(ranks)})")
    if dtype == "bf16":
        p.X_bits = f32_to_bf16_bits(X)
        p.W_bits = f32_to_bf16_bits(W)
        p.A_bits = [f32_to_bf16_bits(a) for a in A]
        p.B_bits = [f32_to_bf16_bits(b) for b in B]
        p.X = bf16_bits_to_f32(p.X_bits)
        p.W = bf16_bits_to_f32(p.W_bits)
        p.A = [bf16_bits_to_f32(a) for a in p.A_bits]
        p.B = [bf16_bits_to_f32(b) for b in p.B_bits]
    return p


# ---------------------------------------------------------------- many adapters in one batch
MIXED_ADAPTERS = 4


def mixed_table(M: int, n_adapters: int = MIXED_ADAPTERS, seed: int = 3):
    """Segments of 20..140 rows, each naming one of n_adapters adapters or none (seeded): the
    many-adapters batch of the 16k-row prefill layer (212 segments at M = 16,384)."""
    g = np.random.Generator(np.random.PCG64(seed))
    starts, labels = [0], []
    while starts[-1] < M:
        starts.append(min(M, starts[-1] + int(g.integers(20, 141))))
        labels.append(int(g.integers(-1, n_adapters)))
    return starts, labels


def extra_adapter_seed(cfg: int, layer: int, proj: int, tensor: int, j: int) -> int:
    """Seed of adapter j >= 1 of a projection in the many-adapters batch (adapter 0 uses seed_of)."""
    return seed_of(cfg, layer, proj, tensor) + 100 * j


# ---------------------------------------------------------------- row samples
def sample_rows(M: int, seg_starts, n: int, seed: int, tiles=(128, 256)) -> np.ndarray:
    """Sorted distinct rows to check when the whole output is too large for the oracle.

    The first and last row of every non-empty segment, the rows on each side of
    tile boundaries (as many as fit in half the budget), then seeded uniform rows.
    """
    if M <= n:
        return np.arange(M, dtype=np.int64)
    chosen = set()
    s = list(seg_starts)
    for a, b in zip(s[:-1], s[1:]):
        if b > a:
            chosen.update((a, b - 1))
    chosen.add(M - 1)
    bound = []
    for t in tiles:
        for m in range(t, M, t):
            bound.extend((m - 1, m))
    g = np.random.Generator(np.random.PCG64(seed))
    if len(bound) > n // 2:
        bound = list(g.choice(np.array(bound), n // 2, replace=False))
    chosen.update(int(b) for b in bound)
    while len(chosen) < n:
        chosen.update(int(v) for v in g.integers(0, M, size=n - len(chosen)))
    out = np.array(sorted(chosen), dtype=np.int64)
    return out[:max(n, 0)] if len(out) > n else out


# ---------------------------------------------------------------- device draws
def device_normal_bf16(shape, sigma: float, seed: int, device="cuda"):
    """bf16 N(0, sigma^2) drawn on the device with torch's seeded generator.

    Used to fill the multi-gigabyte weight stacks the benchmark times; these
    are not the host recipe's values, so parity checks use the host draws.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    t.mul_(sigma)
    return t.to(torch.bfloat16)


# ---------------------------------------------------------------- 4-bit base weights
Q4_GROUP = 128      # weights of one row that share a scale and a zero point, along K


def quantize_q4(W: np.ndarray):
    """Stand-in 4-bit copy of a weight matrix (round to nearest, min/max per group).

    The pages serve a 4-bit copy of the base weights (W4A16) without printing its
    format; this draws one in the common asymmetric form: for each row n and
    group g of 128 consecutive k, a bf16 scale s and an integer zero point z in
    0..15, and codes q in 0..15 with w ~ s (q - z).

    Returns (packed uint8 N x K/2, params uint32 K/128 x N, codes uint8 N x K,
    scale float32 N x K/128, zero int N x K/128).  Packing: code k sits in byte
    k // 2, low nibble for even k, high nibble for odd k.  Params word (g, n):
    bits 0-15 the bf16 scale, bits 16-23 the zero point.
    """
    W = np.asarray(W, dtype=np.float64)
    N, K = W.shape
    if K % Q4_GROUP:
        raise ValueError("K must be a multiple of 128")
    G = K // Q4_GROUP
    Wg = W.reshape(N, G, Q4_GROUP)
    lo = np.minimum(Wg.min(axis=2), 0.0)
    hi = np.maximum(Wg.max(axis=2), 0.0)
    step = (hi - lo) / 15.0
    step[step == 0] = 1.0
    s_bits = f32_to_bf16_bits(step.astype(np.float32))
    s = bf16_bits_to_f32(s_bits).astype(np.float64)
    z = np.clip(np.rint(-lo / s), 0, 15).astype(np.int64)
    q = np.clip(np.rint(Wg / s[:, :, None] + z[:, :, None]), 0, 15).astype(np.uint8).reshape(N, K)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    params = (s_bits.astype(np.uint32) | (z.astype(np.uint32) << 16)).T.copy()
    return packed, params, q, s.astype(np.float32), z


def device_quantize_q4(W):
    """quantize_q4's recipe on a bf16 CUDA tensor (N, K), for the multi-gigabyte weight stacks the
    benchmark times.  Returns (packed uint8 (N, K/2), params int32 (K/128, N)) on the device."""
    import torch
    N, K = W.shape
    G = K // Q4_GROUP
    Wg = W.float().view(N, G, Q4_GROUP)
    lo = Wg.amin(dim=2).clamp(max=0.0)
    hi = Wg.amax(dim=2).clamp(min=0.0)
    step = (hi - lo) / 15.0
    step = torch.where(step == 0, torch.ones_like(step), step)
    s_b = step.to(torch.bfloat16)
    s = s_b.float()
    z = torch.clamp(torch.round(-lo / s), 0, 15)
    q = torch.clamp(torch.round(Wg / s[..., None] + z[..., None]), 0, 15).to(torch.uint8).view(N, K)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).contiguous()
    s_bits = s_b.view(torch.int16).to(torch.int32) & 0xFFFF
    params = (s_bits | (z.to(torch.int32) << 16)).t().contiguous()
    return packed, params
