"""The plain definition of the mixed-adapter LoRA projection, in float64.

Source: "two 27B models on a single RTX 5090" (blog.kvit.app).
  * Section 3, weights figure: each changed matrix of the adapted model is the
    base matrix plus a rank-256 product, W_clef = W_qwen + B.A, with A of shape
    r x K and B of shape N x r.
  * Section 4, request-path figure: a request that names the adapter runs, in
    each changed matrix, the base product plus the output of the adapter's two
    thin matrices applied in turn; a request that names the base model uses the
    base weights alone; both kinds of request share one batch.

So, for a token row x of a request naming adapter a (s_a is that adapter's
scale, 1.0 for the pages' unscaled merge; a call may give one s for every
adapter or one per adapter, since each adapter is its own merge):

    y = x W^T + s_a * ((x A_a^T) B_a^T)

and for every other row y = x W^T.  The rows of one request are contiguous:
segment g covers rows [seg_starts[g], seg_starts[g+1]) and seg_adapter[g] is
its adapter index, or -1 for the base weights alone.

The oracle computes exactly this in float64, one segment at a time, with the
adapter term formed in the order the pages give (shrink by A, then expand by
B).  Inputs are the exact values of the stored elements (bf16 or fp32, widened
to float64 without change); the result stays in float64.  Matrix products use
numpy's float64 matmul as a library step.
"""
from __future__ import annotations

import numpy as np


def validate_segments(seg_starts, seg_adapter, M: int, n_adapters: int):
    """Check that the segments tile rows [0, M) in order and name valid adapters."""
    s = np.asarray(seg_starts, dtype=np.int64)
    a = np.asarray(seg_adapter, dtype=np.int64)
    if s.ndim != 1 or a.ndim != 1 or len(s) != len(a) + 1:
        raise ValueError("seg_starts must have one more entry than seg_adapter")
    if M > 0 and len(a) == 0:
        raise ValueError("a non-empty batch needs at least one segment")
    if len(a) == 0:
        return s, a
    if s[0] != 0 or s[-1] != M or np.any(np.diff(s) < 0):
        raise ValueError("segments must start at 0, never go backwards and end at M")
    if np.any(a < -1) or np.any(a >= n_adapters):
        raise ValueError("adapter index out of range")
    return s, a


def lora_proj_ref(X, seg_starts, seg_adapter, W, A, B, scale, rows=None) -> np.ndarray:
    """Y = X W^T, plus s_a (X A_a^T) B_a^T on the rows of segments naming adapter a.

    X: (M, K), W: (N, K), A: list of (r_a, K), B: list of (N, r_a) — exact
    input values (any float dtype); each adapter may have its own rank r_a.
    scale: one number for every adapter, or a sequence with one per adapter.
    rows: optional global row indices; only those rows of Y are computed (rows
    are independent of one another).
    Returns float64 of shape (len(rows), N).
    """
    X = np.asarray(X)
    M, K = X.shape
    W64 = np.asarray(W, dtype=np.float64)
    N = W64.shape[0]
    if W64.shape[1] != K:
        raise ValueError("W must be N x K")
    s, a = validate_segments(seg_starts, seg_adapter, M, len(A))
    if np.ndim(scale) == 0:
        scales = [float(scale)] * len(A)
    else:
        scales = [float(v) for v in scale]
        if len(scales) != len(A):
            raise ValueError("one scale per adapter")
    rows = np.arange(M, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    Y = np.empty((len(rows), N), dtype=np.float64)
    if len(rows) == 0:
        return Y
    seg_of_row = np.searchsorted(s, rows, side="right") - 1
    for g in np.unique(seg_of_row):
        pos = np.nonzero(seg_of_row == g)[0]
        x = X[rows[pos]].astype(np.float64)
        base = x @ W64.T
        adapter = int(a[g])
        if adapter < 0:
            Y[pos] = base
            continue
        A64 = np.asarray(A[adapter], dtype=np.float64)
        B64 = np.asarray(B[adapter], dtype=np.float64)
        if A64.shape[1] != K or B64.shape[0] != N or A64.shape[0] != B64.shape[1]:
            raise ValueError("A must be r x K and B must be N x r")
        t = x @ A64.T                  # the first thin matrix: r values per row
        Y[pos] = base + scales[adapter] * (t @ B64.T)   # the second, added to the base
    return Y


def lora_proj_sliced_ref(X, seg_starts, seg_adapter, W, A, B, scale, slice_n, rows=None) -> np.ndarray:
    """Several projections of the same rows, their weights concatenated along N.

    "two 27B models on a single RTX 5090", section 4 request-path figure: every
    changed matrix runs the base product plus the adapter's two thin matrices.
    A group of changed matrices that read the same rows (query, key and value;
    gate and up) is stored as one matrix: W is the slices' weights stacked along
    N, each A[a] stacks the slices' first thin matrices ((S r) x K, slice s in
    rows s r .. s r + r - 1) and each B[a] stacks their second ones along N.
    The result is, slice by slice, the plain projection of that slice's own
    W, A and B, with the outputs side by side; the oracle computes exactly that.

    slice_n: the slices' widths (summing to N).  Returns float64 (len(rows), N).
    """
    W = np.asarray(W)
    widths = [int(v) for v in slice_n]
    if any(w < 1 for w in widths) or sum(widths) != W.shape[0]:
        raise ValueError("slice widths must be positive and sum to N")
    S = len(widths)
    outs = []
    c0 = 0
    for s, w in enumerate(widths):
        As, Bs = [], []
        for a in range(len(A)):
            Aa = np.asarray(A[a])
            if Aa.shape[0] % S:
                raise ValueError("A must stack one r x K factor per slice")
            r = Aa.shape[0] // S
            As.append(Aa[s * r:(s + 1) * r])
            Bs.append(np.asarray(B[a])[c0:c0 + w])
        outs.append(lora_proj_ref(X, seg_starts, seg_adapter, W[c0:c0 + w], As, Bs, scale, rows=rows))
        c0 += w
    return np.concatenate(outs, axis=1)


def dequantize_q4(packed, params, K: int) -> np.ndarray:
    """Exact values of a 4-bit weight matrix, float64 (N x K).

    "two 27B models on a single RTX 5090", section 4 memory figure: the card
    holds a 4-bit copy of the base weights beside the bf16 adapter.  The pages
    do not print the format; this library's (W4A16, asymmetric, groups of 128
    along K, as AutoRound writes by default): codes of row n are packed two per byte along K, code k in
    byte k // 2, the low nibble for even k and the high nibble for odd k.  Each
    group g of 128 consecutive k of row n has a params word params[g, n]: bits
    0-15 a bf16 scale s, bits 16-23 a zero point z.  The weight is s (q - z).
    """
    packed = np.asarray(packed, dtype=np.uint8)
    params = np.asarray(params, dtype=np.uint32)
    N = packed.shape[0]
    if packed.shape[1] * 2 != K or K % 128 or params.shape != (K // 128, N):
        raise ValueError("packed must be N x K/2 and params K/128 x N, K a multiple of 128")
    q = np.empty((N, K), dtype=np.float64)
    q[:, 0::2] = packed & 0xF
    q[:, 1::2] = packed >> 4
    scale = ((params & 0xFFFF).astype(np.uint32) << 16).view(np.float32).astype(np.float64).T   # N x G
    zero = ((params >> 16) & 0xFF).astype(np.float64).T
    g = np.arange(K) // 128
    return scale[:, g] * (q - zero[:, g])


def lora_proj_q4_ref(X, seg_starts, seg_adapter, packed, params, A, B, scale, slice_n=None, rows=None):
    """The projection with the base weights given in 4-bit form: W is their exact
    dequantized values (dequantize_q4), and everything else is lora_proj_ref
    (lora_proj_sliced_ref when slice_n is given)."""
    K = np.asarray(X).shape[1]
    W = dequantize_q4(packed, params, K)
    if slice_n is None:
        return lora_proj_ref(X, seg_starts, seg_adapter, W, A, B, scale, rows=rows)
    return lora_proj_sliced_ref(X, seg_starts, seg_adapter, W, A, B, scale, slice_n, rows=rows)
