"""ctypes binding of liblora_proj.so — argument marshalling only.

Every step of the projection runs in the library's HIP kernels.  PyTorch is
used for device memory and streams: tensors hand over their data pointers and
the current stream.  If the library is not built, the first call raises; there
is no other path.
"""
from __future__ import annotations

import ctypes
import numbers
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblora_proj.so")

(LORA_OK, LORA_EINVAL, LORA_ESEGMENTS, LORA_EADAPTER, LORA_EUNSUPPORTED, LORA_EWORKSPACE, LORA_EHIP,
 LORA_EHANDOVER) = range(8)
STATUS_NAMES = {0: "LORA_OK", 1: "LORA_EINVAL", 2: "LORA_ESEGMENTS", 3: "LORA_EADAPTER",
                4: "LORA_EUNSUPPORTED", 5: "LORA_EWORKSPACE", 6: "LORA_EHIP", 7: "LORA_EHANDOVER"}
DTYPES = {"bf16": 0, "f32": 1, "bf16_f32out": 2}
MAX_SEGMENTS, MAX_ADAPTERS, MIN_RANK, MAX_RANK = 256, 32, 16, 512
MAX_SLICES, SLICE_ALIGN = 4, 256
WORKSPACE_COUNTER_BYTES = 65536   # zero-filled counter area at the start of every workspace
EXPORTS = ("lora_proj", "lora_proj_ex", "lora_proj_multi", "lora_proj_sliced", "lora_proj_q4",
           "lora_proj_workspace_bytes", "lora_proj_sliced_workspace_bytes", "lora_proj_q4_workspace_bytes",
           "lora_proj_path", "lora_proj_tile_rows", "lora_status_string", "lora_extract", "lora_extract_workspace_bytes",
           "lora_probe_mfma_bf16", "lora_probe_read", "lora_workspace_status", "lora_debug_handover_fault",
           "lora_decode_plan_describe", "lora_proj_noalloc", "lora_proj_ranked")
NOALLOC_SCRATCH_BYTES = 64 << 20   # the device array lora_proj_noalloc uses instead of a workspace
PLAN_FIELDS = ("MT", "nst", "nrs", "ntA", "ntW", "n_used", "GA", "GW", "smaxW", "off_cnt", "off_pa", "pa_bytes",
               "off_pw", "pw_bytes", "off_th", "t_bytes", "off_tl", "total")

_lib = None


class LoraError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load():
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m rank_adapted_gemm_amd.build`")
    # PyTorch ships its own copy of the HIP runtime with the same soname as the
    # system one.  Importing torch first makes the library bind to that copy;
    # loading the library first would map a second HIP runtime into the
    # process once torch is imported, and the two would share no state.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.lora_proj.argtypes = [vp, i32p, i32p, i32, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i32,
                              ctypes.c_float, vp, i64, i64, i64, ctypes.c_int, vp, sz, vp]
    lib.lora_proj.restype = ctypes.c_int
    lib.lora_proj_ex.argtypes = lib.lora_proj.argtypes + [vp, vp]
    lib.lora_proj_ex.restype = ctypes.c_int
    lib.lora_proj_multi.argtypes = (lib.lora_proj.argtypes[:9] + [ctypes.POINTER(ctypes.c_float)] +
                                    lib.lora_proj.argtypes[10:])
    lib.lora_proj_multi.restype = ctypes.c_int
    lib.lora_proj_sliced.argtypes = (lib.lora_proj_multi.argtypes[:10] + [i32, ctypes.POINTER(i64)] +
                                     lib.lora_proj_multi.argtypes[10:])
    lib.lora_proj_sliced.restype = ctypes.c_int
    lib.lora_proj_ranked.argtypes = (lib.lora_proj_sliced.argtypes[:8] + [i32p] + lib.lora_proj_sliced.argtypes[9:])
    lib.lora_proj_ranked.restype = ctypes.c_int
    lib.lora_proj_sliced_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.c_int]
    lib.lora_proj_sliced_workspace_bytes.restype = sz
    lib.lora_proj_q4.argtypes = lib.lora_proj_sliced.argtypes[:5] + [vp] + lib.lora_proj_sliced.argtypes[5:]
    lib.lora_proj_q4.restype = ctypes.c_int
    lib.lora_proj_q4_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.c_int]
    lib.lora_proj_q4_workspace_bytes.restype = sz
    lib.lora_extract.argtypes = [vp, vp, i64, i64, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.lora_extract.restype = ctypes.c_int
    lib.lora_extract_workspace_bytes.argtypes = [i64, i64, i32, i32]
    lib.lora_extract_workspace_bytes.restype = sz
    lib.lora_probe_mfma_bf16.argtypes = [i32, vp, ctypes.POINTER(ctypes.c_double), vp]
    lib.lora_probe_mfma_bf16.restype = ctypes.c_int
    lib.lora_probe_read.argtypes = [vp, sz, vp, vp]
    lib.lora_probe_read.restype = ctypes.c_int
    lib.lora_proj_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, ctypes.c_int]
    lib.lora_proj_workspace_bytes.restype = sz
    lib.lora_proj_path.argtypes = [i64, i64, i64, i32, ctypes.c_int]
    lib.lora_proj_path.restype = ctypes.c_char_p
    lib.lora_proj_tile_rows.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.lora_proj_tile_rows.restype = i32
    lib.lora_status_string.argtypes = [ctypes.c_int]
    lib.lora_status_string.restype = ctypes.c_char_p
    lib.lora_proj_noalloc.argtypes = lib.lora_proj.argtypes[:15] + [vp]
    lib.lora_proj_noalloc.restype = ctypes.c_int
    lib.lora_workspace_status.argtypes = [vp, sz, vp]
    lib.lora_workspace_status.restype = ctypes.c_int
    lib.lora_debug_handover_fault.argtypes = [i32]
    lib.lora_debug_handover_fault.restype = i32
    lib.lora_decode_plan_describe.argtypes = [i64, i64, i64, i32, i32, ctypes.POINTER(i64), i32,
                                              ctypes.POINTER(i64), i32]
    lib.lora_decode_plan_describe.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().lora_status_string(status).decode()


def workspace_bytes(M: int, N: int, K: int, rank: int, n_adapters: int = 1, dtype: str = "bf16",
                    n_slices: int = 1) -> int:
    if n_slices == 1:
        return int(load().lora_proj_workspace_bytes(M, N, K, rank, n_adapters, DTYPES[dtype]))
    return int(load().lora_proj_sliced_workspace_bytes(M, N, K, rank, n_slices, n_adapters, DTYPES[dtype]))


def q4_workspace_bytes(M: int, N: int, K: int, rank: int, n_adapters: int = 1, dtype: str = "bf16",
                       n_slices: int = 1) -> int:
    return int(load().lora_proj_q4_workspace_bytes(M, N, K, rank, n_slices, n_adapters, DTYPES[dtype]))


def _check_operands(dev, named, shapes=()):
    """Every tensor in ``named`` (name -> tensor) on CUDA device ``dev``, and each
    (name, tensor, shape) in ``shapes`` exactly that shape: the library reads
    operands by pointer and sizes alone, so a mismatch here would be read out of
    bounds on the device."""
    for name, t in named.items():
        if t is not None and (not t.is_cuda or t.device != dev):
            raise ValueError(f"{name} must be a CUDA tensor on {dev}")
    for name, t, shape in shapes:
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream_of(stream, dev):
    """The torch stream a wrapper enqueues on: torch's current stream on ``dev`` when ``stream`` is
    None, else ``stream`` itself, which must be a torch.cuda.Stream (or ExternalStream) on ``dev``.

    The wrappers allocate their output and workspace inside ``torch.cuda.stream(s)``, so the
    workspace's zero-fill is ordered before the kernel on that same stream, and the caching
    allocator hands a freed block only to later work on that stream (which runs after the kernel).
    Raw stream handles go through the *_raw functions, which allocate nothing."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(dev)
    if not isinstance(stream, torch.cuda.Stream):
        raise TypeError("stream must be a torch.cuda.Stream (raw hipStream_t handles go through the *_raw "
                        "functions, which allocate nothing)")
    if stream.device != dev:
        raise ValueError(f"stream is on {stream.device}, the operands on {dev}")
    return stream


def lora_proj_q4_raw(X, seg_starts, seg_adapter, Wq, Wp, A, B, rank, scales, Y, M, N, K, dtype,
                     workspace=None, workspace_bytes_=0, stream=None, slices=None) -> int:
    """lora_proj_q4 with raw device addresses (ints); ``scales`` one float per adapter."""
    lib = load()
    starts = (ctypes.c_int32 * len(seg_starts))(*[int(v) for v in seg_starts])
    adapt = (ctypes.c_int32 * max(len(seg_adapter), 1))(*[int(v) for v in seg_adapter])
    n_ad = len(A)
    a_arr = (ctypes.c_void_p * max(n_ad, 1))(*[ctypes.c_void_p(a) if a else None for a in A])
    b_arr = (ctypes.c_void_p * max(n_ad, 1))(*[ctypes.c_void_p(b) if b else None for b in B])
    if isinstance(scales, numbers.Real):
        scales = [float(scales)] * n_ad
    if len(scales) != n_ad:
        raise ValueError("one scale per adapter")
    s_arg = (ctypes.c_float * max(n_ad, 1))(*[float(v) for v in scales])
    widths = list(slices) if slices is not None else [int(N)]
    w_arg = (ctypes.c_int64 * len(widths))(*[int(v) for v in widths])
    return int(lib.lora_proj_q4(X, starts, adapt, len(seg_adapter), Wq, Wp, a_arr, b_arr, n_ad, int(rank), s_arg,
                                len(widths), w_arg, Y, int(M), int(N), int(K),
                                DTYPES[dtype] if isinstance(dtype, str) else int(dtype), workspace,
                                int(workspace_bytes_), stream))


def lora_proj_q4(X, seg_starts, seg_adapter, Wq, Wp, A, B, scale, out=None, workspace=None, dtype="bf16",
                 stream=None, slices=None):
    """Y with the base weights in 4-bit form: Wq (N, K/2) uint8 codes, Wp (K/128, N) int32 params words.

    Other arguments as lora_proj; returns Y (M, N).
    """
    import torch
    M, K = X.shape
    N = Wq.shape[0]
    for t in (X, *A, *B):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("X, A, B must be contiguous bfloat16 CUDA tensors")
    s = _stream_of(stream, X.device)
    for t in (Wq, Wp):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("Wq and Wp must be contiguous CUDA tensors")
    n_slices = 1 if slices is None else len(slices)
    rank = A[0].shape[0] // n_slices if len(A) else 0
    out_t = torch.bfloat16 if dtype == "bf16" else torch.float32
    if out is None:
        with torch.cuda.stream(s):
            out = torch.empty((M, N), dtype=out_t, device=X.device)
    if out.dtype != out_t or not out.is_contiguous():
        raise ValueError("out must be a contiguous (M, N) tensor of the output dtype")
    _check_operands(X.device, {"Wq": Wq, "Wp": Wp, "out": out, "workspace": workspace,
                               **{f"A[{i}]": a for i, a in enumerate(A)}, **{f"B[{i}]": b for i, b in enumerate(B)}},
                    [("Wq", Wq, (N, K // 2)), ("Wp", Wp, ((K + 127) // 128, N)), ("out", out, (M, N))]
                    + [(f"A[{i}]", a, (n_slices * rank, K)) for i, a in enumerate(A)]
                    + [(f"B[{i}]", b, (N, rank)) for i, b in enumerate(B)])
    if Wq.element_size() * Wq.shape[1] != K // 2 or Wp.element_size() != 4:
        raise ValueError("Wq holds K/2 bytes per row and Wp 32-bit words")
    need = q4_workspace_bytes(M, N, K, rank if len(A) else 16, len(A), dtype, n_slices)
    if workspace is None and need:
        with torch.cuda.stream(s):   # zero-filled on the call's stream: the counter area starts at zero
            workspace = torch.zeros(need, dtype=torch.uint8, device=X.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lora_proj_q4_raw(X.data_ptr(), seg_starts, seg_adapter, Wq.data_ptr(), Wp.data_ptr(),
                          [a.data_ptr() for a in A], [b.data_ptr() for b in B], rank, scale, out.data_ptr(),
                          M, N, K, dtype, ws_ptr, ws_bytes, s.cuda_stream, slices)
    if st != LORA_OK:
        raise LoraError(st, status_string(st))
    return out


def extract_workspace_bytes(N: int, K: int, l: int, rank: int) -> int:
    return int(load().lora_extract_workspace_bytes(N, K, l, rank))


def extract_raw(Wa, Wb, N, K, omega, l, rank, power_iters, B, A, sigma, workspace, workspace_bytes_, stream=None):
    """lora_extract with raw device addresses (ints).  Returns the status code."""
    return int(load().lora_extract(Wa, Wb, int(N), int(K), omega, int(l), int(rank), int(power_iters), B, A, sigma,
                                   workspace, int(workspace_bytes_), stream))


def extract(W_adapted, W_base, rank, omega, power_iters=2, stream=None):
    """(B (N, r), A (r, K), sigma (r,)) fp32 CUDA tensors: the rank-r truncated SVD of
    W_adapted - W_base (bf16 CUDA tensors, N x K), with omega the K x l fp32 Gaussian test matrix."""
    import torch
    N, K = W_adapted.shape
    l = omega.shape[1]
    for t in (W_adapted, W_base):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("weights must be contiguous bfloat16 CUDA tensors")
    if omega.dtype != torch.float32 or not omega.is_contiguous() or omega.dim() != 2 or omega.shape[0] != K:
        raise ValueError("omega must be a contiguous float32 K x l tensor")
    dev = W_adapted.device
    _check_operands(dev, {"W_base": W_base, "omega": omega}, [("W_base", W_base, (N, K))])
    s = _stream_of(stream, dev)
    need = extract_workspace_bytes(N, K, l, rank)
    with torch.cuda.stream(s):
        B = torch.empty((N, rank), dtype=torch.float32, device=dev)
        A = torch.empty((rank, K), dtype=torch.float32, device=dev)
        sigma = torch.empty((rank,), dtype=torch.float32, device=dev)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = extract_raw(W_adapted.data_ptr(), W_base.data_ptr(), N, K, omega.data_ptr(), l, rank, power_iters,
                     B.data_ptr(), A.data_ptr(), sigma.data_ptr(), ws.data_ptr(), need, s.cuda_stream)
    if st != LORA_OK:
        raise LoraError(st, status_string(st))
    return B, A, sigma


def path(M: int, N: int, K: int, rank: int, dtype: str = "bf16") -> str:
    return load().lora_proj_path(M, N, K, rank, DTYPES[dtype]).decode()


def tile_rows(M: int, N: int, K: int, dtype: str = "bf16") -> int:
    """Activation rows per prefill output tile for this shape (0 off the prefill path)."""
    return int(load().lora_proj_tile_rows(M, N, K, DTYPES[dtype]))


def lora_proj_raw(X, seg_starts, seg_adapter, W, A, B, rank, scale, Y, M, N, K, dtype,
                  workspace=None, workspace_bytes_=0, stream=None, events=None, slices=None) -> int:
    """Call the C entry point with raw device addresses (ints) and host segment lists.

    ``events``: optional (start, stop) hipEvent_t handles recorded around the
    output kernel (calls lora_proj_ex).  ``scale``: one float for every adapter,
    or a sequence with one scale per adapter (calls lora_proj_multi, which takes
    no events).  ``slices``: output-column widths of a sliced call (calls
    lora_proj_sliced; A[a] then holds the slices' factors stacked, S*rank rows).
    Returns the status code.
    """
    lib = load()
    starts = (ctypes.c_int32 * len(seg_starts))(*[int(v) for v in seg_starts])
    adapt = (ctypes.c_int32 * max(len(seg_adapter), 1))(*[int(v) for v in seg_adapter])
    n_ad = len(A)
    a_arr = (ctypes.c_void_p * max(n_ad, 1))(*[ctypes.c_void_p(a) if a else None for a in A])
    b_arr = (ctypes.c_void_p * max(n_ad, 1))(*[ctypes.c_void_p(b) if b else None for b in B])
    per_adapter = not isinstance(scale, numbers.Real) or slices is not None
    if per_adapter and isinstance(scale, numbers.Real):
        scale = [float(scale)] * n_ad
    if per_adapter:
        scales = [float(v) for v in scale]
        if len(scales) != n_ad:
            raise ValueError("one scale per adapter")
        if events is not None:
            raise ValueError("per-adapter scales take no timing events")
        s_arg = (ctypes.c_float * max(n_ad, 1))(*scales)
    else:
        s_arg = float(scale)
    args = (X, starts, adapt, len(seg_adapter), W, a_arr, b_arr, n_ad, int(rank), s_arg, Y,
            int(M), int(N), int(K), DTYPES[dtype] if isinstance(dtype, str) else int(dtype),
            workspace, int(workspace_bytes_), stream)
    if slices is not None:
        widths = (ctypes.c_int64 * max(len(slices), 1))(*[int(v) for v in slices])
        return int(lib.lora_proj_sliced(*args[:10], len(slices), widths, *args[10:]))
    if per_adapter:
        return int(lib.lora_proj_multi(*args))
    if events is not None:
        return int(lib.lora_proj_ex(*args, events[0], events[1]))
    return int(lib.lora_proj(*args))


def lora_proj(X, seg_starts, seg_adapter, W, A, B, scale, out=None, workspace=None, dtype=None, stream=None,
              events=None, slices=None):
    """Y = X W^T, plus s (X A_a^T) B_a^T on rows of segments naming adapter a.

    ``scale`` is one float, or a sequence of one scale per adapter.  ``slices``:
    widths of the output-column slices of a sliced call (A[a] is then
    (len(slices) * r, K), slice s's factor in rows s r .. s r + r - 1).
    X (M, K), W (N, K), A[a] (r, K), B[a] (N, r): contiguous CUDA tensors of one
    dtype (bfloat16, or float32 for the test mode).  seg_starts / seg_adapter:
    host sequences of ints.  dtype: "bf16", "f32" or "bf16_f32out" (default
    from X).  Returns Y (M, N); raises LoraError on a non-OK status.
    """
    import torch
    if dtype is None:
        dtype = "f32" if X.dtype == torch.float32 else "bf16"
    in_t = torch.float32 if dtype == "f32" else torch.bfloat16
    out_t = torch.bfloat16 if dtype == "bf16" else torch.float32
    tensors = [X, W, *A, *B]
    for t in tensors:
        if t.dtype != in_t or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"inputs must be contiguous {in_t} CUDA tensors")
    M, K = X.shape
    N = W.shape[0]
    n_slices = 1 if slices is None else len(slices)
    rank = A[0].shape[0] // n_slices if len(A) else 0
    s = _stream_of(stream, X.device)
    if out is None:
        with torch.cuda.stream(s):
            out = torch.empty((M, N), dtype=out_t, device=X.device)
    if out.dtype != out_t or not out.is_contiguous() or tuple(out.shape) != (M, N):
        raise ValueError("out must be a contiguous (M, N) tensor of the output dtype")
    _check_operands(X.device, {"W": W, "out": out, "workspace": workspace,
                               **{f"A[{i}]": a for i, a in enumerate(A)}, **{f"B[{i}]": b for i, b in enumerate(B)}},
                    [("W", W, (N, K))]
                    + [(f"A[{i}]", a, (n_slices * rank, K)) for i, a in enumerate(A)]
                    + [(f"B[{i}]", b, (N, rank)) for i, b in enumerate(B)])
    need = workspace_bytes(M, N, K, rank if len(A) else 16, len(A), dtype, n_slices)
    if workspace is None and need:
        with torch.cuda.stream(s):   # zero-filled on the call's stream: the counter area starts at zero
            workspace = torch.zeros(need, dtype=torch.uint8, device=X.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lora_proj_raw(X.data_ptr(), seg_starts, seg_adapter, W.data_ptr(),
                       [a.data_ptr() for a in A], [b.data_ptr() for b in B], rank, scale,
                       out.data_ptr(), M, N, K, dtype, ws_ptr, ws_bytes, s.cuda_stream, events, slices)
    if st != LORA_OK:
        raise LoraError(st, status_string(st))
    return out


def lora_proj_ranked_raw(X, seg_starts, seg_adapter, W, A, B, ranks, scales, Y, M, N, K, dtype, workspace=None,
                         workspace_bytes_=0, stream=None, slices=None) -> int:
    """lora_proj_ranked with raw device addresses (ints): one rank and one scale per adapter.
    Returns the status code."""
    lib = load()
    starts = (ctypes.c_int32 * len(seg_starts))(*[int(v) for v in seg_starts])
    adapt = (ctypes.c_int32 * max(len(seg_adapter), 1))(*[int(v) for v in seg_adapter])
    n_ad = len(A)
    if len(ranks) != n_ad or len(scales) != n_ad:
        raise ValueError("one rank and one scale per adapter")
    a_arr = (ctypes.c_void_p * max(n_ad, 1))(*[ctypes.c_void_p(a) if a else None for a in A])
    b_arr = (ctypes.c_void_p * max(n_ad, 1))(*[ctypes.c_void_p(b) if b else None for b in B])
    r_arg = (ctypes.c_int32 * max(n_ad, 1))(*[int(v) for v in ranks])
    s_arg = (ctypes.c_float * max(n_ad, 1))(*[float(v) for v in scales])
    widths = list(slices) if slices is not None else [int(N)]
    w_arg = (ctypes.c_int64 * len(widths))(*[int(v) for v in widths])
    return int(lib.lora_proj_ranked(X, starts, adapt, len(seg_adapter), W, a_arr, b_arr, n_ad, r_arg, s_arg,
                                    len(widths), w_arg, Y, int(M), int(N), int(K),
                                    DTYPES[dtype] if isinstance(dtype, str) else int(dtype), workspace,
                                    int(workspace_bytes_), stream))


def lora_proj_ranked(X, seg_starts, seg_adapter, W, A, B, scales, out=None, workspace=None, dtype=None, stream=None,
                     slices=None):
    """lora_proj with each adapter at its own rank r_a, read from its factors: A[a] is
    (len(slices) * r_a, K) (slice s's factor in rows s r_a .. s r_a + r_a - 1), B[a] is (N, r_a).
    ``scales``: one float per adapter.  Returns Y (M, N); raises LoraError on a non-OK status."""
    import torch
    if dtype is None:
        dtype = "f32" if X.dtype == torch.float32 else "bf16"
    in_t = torch.float32 if dtype == "f32" else torch.bfloat16
    out_t = torch.bfloat16 if dtype == "bf16" else torch.float32
    for t in [X, W, *A, *B]:
        if t.dtype != in_t or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"inputs must be contiguous {in_t} CUDA tensors")
    M, K = X.shape
    N = W.shape[0]
    n_slices = 1 if slices is None else len(slices)
    ranks = [int(a.shape[0]) // n_slices for a in A]
    s = _stream_of(stream, X.device)
    if out is None:
        with torch.cuda.stream(s):
            out = torch.empty((M, N), dtype=out_t, device=X.device)
    if out.dtype != out_t or not out.is_contiguous() or tuple(out.shape) != (M, N):
        raise ValueError("out must be a contiguous (M, N) tensor of the output dtype")
    _check_operands(X.device, {"W": W, "out": out, "workspace": workspace,
                               **{f"A[{i}]": a for i, a in enumerate(A)}, **{f"B[{i}]": b for i, b in enumerate(B)}},
                    [("W", W, (N, K))]
                    + [(f"A[{i}]", a, (n_slices * r, K)) for i, (a, r) in enumerate(zip(A, ranks))]
                    + [(f"B[{i}]", b, (N, r)) for i, (b, r) in enumerate(zip(B, ranks))])
    used = {int(a) for a in seg_adapter if int(a) >= 0}
    rmax = max([ranks[a] for a in used], default=16)
    need = workspace_bytes(M, N, K, rmax, len(A), dtype, n_slices)
    if workspace is None and need:
        with torch.cuda.stream(s):   # zero-filled on the call's stream: the counter area starts at zero
            workspace = torch.zeros(need, dtype=torch.uint8, device=X.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lora_proj_ranked_raw(X.data_ptr(), seg_starts, seg_adapter, W.data_ptr(), [a.data_ptr() for a in A],
                              [b.data_ptr() for b in B], ranks, scales, out.data_ptr(), M, N, K, dtype, ws_ptr,
                              ws_bytes, s.cuda_stream, slices)
    if st != LORA_OK:
        raise LoraError(st, status_string(st))
    return out


def probe_mfma_bf16_raw(iters: int, sink: int, stream=None):
    """Launch the dense-MFMA probe (lora_probe.h).  Returns (status, flop it performs)."""
    flop = ctypes.c_double(0.0)
    st = int(load().lora_probe_mfma_bf16(int(iters), sink, ctypes.byref(flop), stream))
    return st, flop.value


def probe_read_raw(src: int, nbytes: int, sink: int, stream=None) -> int:
    """Launch the streaming-read probe (lora_probe.h) over nbytes at src.  Returns the status."""
    return int(load().lora_probe_read(src, int(nbytes), sink, stream))


def workspace_status(workspace, stream=None) -> int:
    """lora_workspace_status on a workspace tensor: LORA_OK, or LORA_EHANDOVER when a decode call on
    it lost a hand-over since the last query (the bits are cleared).  Synchronizes the stream."""
    import torch
    s = _stream_of(stream, workspace.device)
    return int(load().lora_workspace_status(workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                            s.cuda_stream))


def debug_handover_fault(on: bool) -> bool:
    """Test hook: while on, decode calls with adapter rows lose their hand-over (see the header)."""
    return bool(load().lora_debug_handover_fault(1 if on else 0))


def decode_plan(M: int, N: int, K: int, rank: int, n_used: int, slices=None) -> dict | None:
    """The decode launch plan of a shape (lora_decode_plan_describe), or None off the decode path."""
    widths = list(slices) if slices is not None else [int(N)]
    w_arg = (ctypes.c_int64 * len(widths))(*[int(v) for v in widths])
    out = (ctypes.c_int64 * 32)()
    n = int(load().lora_decode_plan_describe(int(M), int(N), int(K), int(rank), len(widths), w_arg, int(n_used),
                                             out, 32))
    if n == 0:
        return None
    return dict(zip(PLAN_FIELDS, list(out[:n])))


def lora_proj_noalloc_raw(X, seg_starts, seg_adapter, W, A, B, rank, scale, Y, M, N, K, dtype, stream=None) -> int:
    """lora_proj_noalloc with raw device addresses (ints): lora_proj_raw without the workspace.
    Returns the status code."""
    lib = load()
    starts = (ctypes.c_int32 * len(seg_starts))(*[int(v) for v in seg_starts])
    adapt = (ctypes.c_int32 * max(len(seg_adapter), 1))(*[int(v) for v in seg_adapter])
    n_ad = len(A)
    a_arr = (ctypes.c_void_p * max(n_ad, 1))(*[ctypes.c_void_p(a) if a else None for a in A])
    b_arr = (ctypes.c_void_p * max(n_ad, 1))(*[ctypes.c_void_p(b) if b else None for b in B])
    return int(lib.lora_proj_noalloc(X, starts, adapt, len(seg_adapter), W, a_arr, b_arr, n_ad, int(rank),
                                     float(scale), Y, int(M), int(N), int(K),
                                     DTYPES[dtype] if isinstance(dtype, str) else int(dtype), stream))


def lora_proj_noalloc(X, seg_starts, seg_adapter, W, A, B, scale, out, dtype=None, stream=None):
    """lora_proj through the entry point that allocates nothing: the caller passes `out` (M, N) as
    well as the inputs, and the library's fixed device array serves as the workspace."""
    import torch
    if dtype is None:
        dtype = "f32" if X.dtype == torch.float32 else "bf16"
    in_t = torch.float32 if dtype == "f32" else torch.bfloat16
    out_t = torch.bfloat16 if dtype == "bf16" else torch.float32
    for t in (X, W, *A, *B):
        if t.dtype != in_t or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"inputs must be contiguous {in_t} CUDA tensors")
    M, K = X.shape
    N = W.shape[0]
    rank = A[0].shape[0] if len(A) else 0
    if out.dtype != out_t or not out.is_contiguous() or tuple(out.shape) != (M, N):
        raise ValueError("out must be a contiguous (M, N) tensor of the output dtype")
    _check_operands(X.device, {"W": W, "out": out, **{f"A[{i}]": a for i, a in enumerate(A)},
                               **{f"B[{i}]": b for i, b in enumerate(B)}},
                    [("W", W, (N, K))] + [(f"A[{i}]", a, (rank, K)) for i, a in enumerate(A)]
                    + [(f"B[{i}]", b, (N, rank)) for i, b in enumerate(B)])
    s = _stream_of(stream, X.device)
    st = lora_proj_noalloc_raw(X.data_ptr(), seg_starts, seg_adapter, W.data_ptr(), [a.data_ptr() for a in A],
                               [b.data_ptr() for b in B], rank, scale, out.data_ptr(), M, N, K, dtype, s.cuda_stream)
    if st != LORA_OK:
        raise LoraError(st, status_string(st))
    return out