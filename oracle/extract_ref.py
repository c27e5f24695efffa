"""The adapter hidden in a weight change, in float64 — TEST INFRASTRUCTURE (see oracle/__init__.py).

Source: "two 27B models on a single RTX 5090" (blog.kvit.app), TL;DR: comparing
the adapted model's weights with the base model's shows a change with the
shape of a merged rank-256 LoRA fine-tune, which factored back out is an
adapter vLLM applies per request.  The same page's §7 notes another project
that recovers the same change as an adapter.  The pages do not give the
method; the plainest reading is a truncated singular value decomposition of
the change, which by the Eckart-Young theorem gives the closest rank-r
product in the Frobenius norm:

    D = W_adapted - W_base = U S V^T,    B = U_r S_r^(1/2),    A = S_r^(1/2) V_r^T

so that B A = U_r S_r V_r^T.  The factors are split evenly (column i of B and
row i of A both have norm sqrt(s_i)).  numpy's float64 SVD is the library step.
"""
from __future__ import annotations

import numpy as np


def extract_ref(W_adapted, W_base, rank: int):
    """(B (N x r), A (r x K), s (r,)) of the change W_adapted - W_base, float64.

    Inputs are the exact stored values (any float dtype); the difference is
    formed in float64.  s holds the r largest singular values, descending.
    """
    D = np.asarray(W_adapted, dtype=np.float64) - np.asarray(W_base, dtype=np.float64)
    if D.ndim != 2 or not 1 <= rank <= min(D.shape):
        raise ValueError("rank must be between 1 and min(N, K)")
    U, s, Vt = np.linalg.svd(D, full_matrices=False)
    root = np.sqrt(s[:rank])
    return U[:, :rank] * root, root[:, None] * Vt[:rank], s[:rank].copy()
