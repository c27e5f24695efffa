"""Adapter extraction on the GPU (lora_extract) against the fp64 truncated-SVD oracle.

The change is planted: W_adapted = bf16(W_base + B0 A0) with B0, A0 Gaussian of rank r, so D has a
gap of about three orders of magnitude after its r-th singular value (the rest is bf16 rounding).
The oracle is the exact truncated SVD of the bf16 values' difference.  Bars (relative, Frobenius):
the product B A within 1e-4 of the oracle's (fp32 products over K terms give ~1e-6; the randomized
range with two power iterations adds ~(1e-3)^5), the singular values within 1e-4, and the even split
(column norms of B equal sqrt(sigma)) within 1e-4.
"""
from __future__ import annotations

import numpy as np
import pytest

from gpu_util import log
from oracle import extract_ref
from rank_adapted_gemm_amd import binding as bd
from rank_adapted_gemm_amd import synth

pytestmark = pytest.mark.gpu


def planted_pair(seed, N, K, r):
    g = np.random.Generator(np.random.PCG64(seed))
    Wb = g.standard_normal((N, K), dtype=np.float32) * np.float32(0.14)
    B0 = g.standard_normal((N, r), dtype=np.float32) * np.float32(0.3)
    A0 = g.standard_normal((r, K), dtype=np.float32) * np.float32(0.3)
    wb_bits = synth.f32_to_bf16_bits(Wb)
    wa_bits = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(wb_bits) + B0 @ A0)
    return wa_bits, wb_bits


@pytest.mark.parametrize("N,K,r,l", [(768, 1024, 32, 48), (2048, 5120, 256, 272)])
def test_extract_planted(N, K, r, l):
    import torch
    wa_bits, wb_bits = planted_pair(91, N, K, r)
    dev = lambda b: torch.from_numpy(b.view(np.int16)).to("cuda").view(torch.bfloat16)
    omega = np.random.Generator(np.random.PCG64(92)).standard_normal((K, l), dtype=np.float32)
    log(f"case extract planted N={N} K={K} r={r} l={l}")
    B, A, s = bd.extract(dev(wa_bits), dev(wb_bits), r, torch.from_numpy(omega).to("cuda"), power_iters=2)
    torch.cuda.synchronize()
    B, A, s = (t.double().cpu().numpy() for t in (B, A, s))
    Bo, Ao, so = extract_ref(synth.bf16_bits_to_f32(wa_bits), synth.bf16_bits_to_f32(wb_bits), r)
    P, Po = B @ A, Bo @ Ao
    err = np.linalg.norm(P - Po) / np.linalg.norm(Po)
    serr = np.max(np.abs(s - so) / so)
    split = np.max(np.abs(np.linalg.norm(B, axis=0) - np.sqrt(s)) / np.sqrt(s))
    log(f"  product err {err:.2e}  sigma err {serr:.2e}  split err {split:.2e}  sigma_r/sigma_1 {so[-1] / so[0]:.3f}")
    assert np.all(np.isfinite(P)) and err <= 1e-4 and serr <= 1e-4 and split <= 1e-4


def test_extract_rank_one_exact_direction():
    """A rank-1 change a b^T with small integer entries: sigma_1 = |a| |b| and B A = a b^T."""
    import torch
    N, K, l = 256, 384, 8
    g = np.random.Generator(np.random.PCG64(93))
    a = g.integers(-3, 4, size=N).astype(np.float32)
    b = g.integers(-3, 4, size=K).astype(np.float32)
    wb = synth.f32_to_bf16_bits(np.zeros((N, K), np.float32))
    wa = synth.f32_to_bf16_bits(np.outer(a, b).astype(np.float32))
    dev = lambda bits: torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    omega = torch.from_numpy(g.standard_normal((K, l), dtype=np.float32)).to("cuda")
    B, A, s = bd.extract(dev(wa), dev(wb), 1, omega, power_iters=1)
    torch.cuda.synchronize()
    P = (B.double() @ A.double()).cpu().numpy()
    assert abs(float(s[0]) - np.linalg.norm(a) * np.linalg.norm(b)) <= 1e-5 * np.linalg.norm(a) * np.linalg.norm(b)
    assert np.linalg.norm(P - np.outer(a, b)) <= 1e-5 * np.linalg.norm(np.outer(a, b))


def _int_low_rank(seed, N, K, true_rank):
    """W_adapted = an integer rank-`true_rank` product (entries up to 45, exact in bf16), W_base = 0."""
    g = np.random.Generator(np.random.PCG64(seed))
    B0 = g.integers(-3, 4, size=(N, true_rank)).astype(np.float32)
    A0 = g.integers(-3, 4, size=(true_rank, K)).astype(np.float32)
    D = B0 @ A0
    assert np.abs(D).max() <= 256
    return synth.f32_to_bf16_bits(D), synth.f32_to_bf16_bits(np.zeros_like(D)), D.astype(np.float64)


@pytest.mark.parametrize("N,K,true_rank,r,l,iters", [
    (300, 200, 5, 8, 16, 2),      # rank below r: the extra directions come back with zero singular values
    (130, 72, 16, 16, 16, 0),     # no oversampling, no power iteration, ragged tiles (130 rows: a 2-row tail)
    (72, 130, 16, 16, 18, 1),     # N < K, ragged
])
def test_extract_exact_low_rank(N, K, true_rank, r, l, iters):
    import torch
    wa, wb, D = _int_low_rank(94 + N, N, K, true_rank)
    dev = lambda bits: torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    omega = np.random.Generator(np.random.PCG64(95)).standard_normal((K, l), dtype=np.float32)
    log(f"case extract exact low rank N={N} K={K} true_rank={true_rank} r={r} l={l} iters={iters}")
    B, A, s = bd.extract(dev(wa), dev(wb), r, torch.from_numpy(omega).to("cuda"), power_iters=iters)
    torch.cuda.synchronize()
    B, A, s = (t.double().cpu().numpy() for t in (B, A, s))
    _, _, so = extract_ref(D, np.zeros_like(D), min(r, true_rank))
    err = np.linalg.norm(B @ A - D) / np.linalg.norm(D)
    kept = min(r, true_rank)
    serr = np.max(np.abs(s[:kept] - so) / so)
    tail = np.max(s[kept:]) / s[0] if r > kept else 0.0
    log(f"  product err {err:.2e}  sigma err {serr:.2e}  tail {tail:.2e}")
    assert np.all(np.isfinite(B)) and np.all(np.isfinite(A))
    assert err <= 1e-5 and serr <= 1e-5 and tail <= 1e-5
    assert np.all(np.diff(s) <= 0)


def test_extract_unchanged_matrix():
    """A matrix the fine-tune left alone (W_adapted = W_base): D = 0, so the truncated SVD is zero and
    B, A and the singular values come back exactly zero, with no NaN from the empty range."""
    import torch
    N, K, r, l = 200, 320, 8, 16
    g = np.random.Generator(np.random.PCG64(96))
    wb = synth.f32_to_bf16_bits(g.standard_normal((N, K), dtype=np.float32))
    dev = lambda bits: torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    omega = np.random.Generator(np.random.PCG64(97)).standard_normal((K, l), dtype=np.float32)
    log(f"case extract unchanged matrix N={N} K={K} r={r} l={l}")
    B, A, s = bd.extract(dev(wb), dev(wb.copy()), r, torch.from_numpy(omega).to("cuda"), power_iters=2)
    torch.cuda.synchronize()
    B, A, s = (t.double().cpu().numpy() for t in (B, A, s))
    _, _, so = extract_ref(synth.bf16_bits_to_f32(wb), synth.bf16_bits_to_f32(wb), r)
    assert np.all(so == 0)
    assert np.all(B == 0) and np.all(A == 0) and np.all(s == 0)


def test_binding_refuses_host_or_mismatched_operands():
    """Operands the library would read by pointer and size alone: a host omega, a base matrix of the
    wrong shape and a host output are refused before anything is launched."""
    import torch
    from rank_adapted_gemm_amd import binding
    wa = torch.zeros((64, 96), dtype=torch.bfloat16, device="cuda")
    omega = torch.zeros((96, 16), dtype=torch.float32)
    with pytest.raises(ValueError, match="CUDA"):
        bd.extract(wa, wa.clone(), 8, omega)
    with pytest.raises(ValueError, match="shape"):
        bd.extract(wa, wa[:63].contiguous(), 8, omega.cuda())
    X = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="CUDA"):
        binding.lora_proj(X, [0, 4], [-1], wa, [], [], 1.0, out=torch.zeros((4, 64), dtype=torch.bfloat16))
