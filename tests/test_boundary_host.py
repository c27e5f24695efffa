"""Host-side checks of the C-ABI boundary (no GPU needed).

Every call below is rejected during argument checking, before any HIP call,
so the pointers are placeholders that are never dereferenced.  M == 0 is the
one accepted call, and it launches nothing.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from rank_adapted_gemm_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20          # 16-byte aligned placeholder addresses, never dereferenced
FAKE2, FAKE3, FAKE4, FAKE5 = FAKE * 64, FAKE * 128, FAKE * 192, FAKE * 256


def declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(lora_\w+)\s*\(", text, flags=re.M)
    return names


def test_library_exports_every_declared_function():
    lib = bd.load()
    names = declared_functions()
    assert set(names) == set(bd.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_one_hip_runtime_in_process():
    """The library binds to the HIP runtime torch loaded; no second runtime gets mapped."""
    bd.load()
    import torch  # noqa: F401
    maps = {l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l}
    assert len(maps) == 1, maps


def test_limits_match_header():
    text = open(os.path.join(ROOT, "include", "lora_proj.h")).read()
    for name, val in (("LORA_MAX_SEGMENTS", bd.MAX_SEGMENTS), ("LORA_MAX_ADAPTERS", bd.MAX_ADAPTERS),
                      ("LORA_MIN_RANK", bd.MIN_RANK), ("LORA_MAX_RANK", bd.MAX_RANK),
                      ("LORA_WORKSPACE_COUNTER_BYTES", bd.WORKSPACE_COUNTER_BYTES)):
        assert re.search(rf"#define {name} {val}\b", text), name


def test_status_strings():
    for s in range(8):
        assert bd.status_string(s)
    assert bd.status_string(99) == "unknown status"


def test_workspace_and_path_queries():
    C = bd.WORKSPACE_COUNTER_BYTES
    assert bd.workspace_bytes(16384, 5120, 5120, 256) == C + 16384 * 256 * 4   # prefill: counters + s X A^T
    assert bd.workspace_bytes(16384, 5120, 5120, 256, 0) == 0                  # prefill, base only
    # a small shrink grid (2054 rows: 17 x 2 tiles of 128) splits K = 5120 in 7 (256 // 34), with
    # 64 KiB of fp32 partials per (tile, split) after T, the tiles bounded by 2 x (17 + 1 adapter)
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert bd.workspace_bytes(2054, 5120, 5120, 256) == r256(C + 2054 * 256 * 4) + 7 * 2 * 18 * 65536
    assert bd.workspace_bytes(2054, 5120, 17408, 256, 2) == r256(C + 2054 * 256 * 4) + 7 * 2 * 19 * 65536
    assert bd.workspace_bytes(2054, 5120, 448, 256) == C + 2054 * 256 * 4     # 7 stages of K: no split
    assert bd.workspace_bytes(2054, 5120, 5120, 256, 1, "f32") == C + 2054 * 256 * 4
    assert bd.workspace_bytes(70, 17408, 5120, 256, dtype="f32") == C + 70 * 256 * 4
    assert bd.workspace_bytes(64, 512, 250, 16) == 0          # K not a multiple of 8
    assert bd.workspace_bytes(64, 512, 256, 24) == 0          # rank not a multiple of 16
    # decode (<= 128 rows): split-K partials of W always, plus adapter partials and T
    base = bd.workspace_bytes(70, 5120, 5120, 256, 0)
    one = bd.workspace_bytes(70, 5120, 5120, 256, 1)
    two = bd.workspace_bytes(70, 5120, 5120, 256, 2)
    assert 0 < base < one < two and base % 256 == 0 and base >= C + 70 * 5120 * 4
    # decode counters (one per 128 output columns, plus three) must fit the counter area below the
    # 8 bytes of error bits
    n_fit = ((C - 8) // 8 - 3) * 128
    assert bd.path(70, n_fit, 8, 16) == "decode" and bd.workspace_bytes(70, n_fit, 8, 16) > 0
    assert bd.path(70, n_fit + 128, 8, 16) == "invalid" and bd.workspace_bytes(70, n_fit + 128, 8, 16) == 0
    assert bd.path(200, n_fit + 128, 8, 16) == "prefill"
    assert bd.path(16384, 5120, 5120, 256) == "prefill"
    assert bd.path(70, 5120, 5120, 256) == "decode"
    assert bd.path(128, 5120, 5120, 256) == "decode"
    assert bd.path(129, 5120, 5120, 256) == "prefill"
    assert bd.path(64, 512, 256, 16, "f32") == "f32"
    assert bd.path(64, 512, 252, 16) == "invalid"


def test_tile_rows_choice():
    """The prefill output kernel's tile height: the fewest whole waves of tile times over 256 CUs."""
    assert bd.tile_rows(16384, 5120, 5120) == 256      # 1,280 tiles of 256 rows: 5 full waves
    assert bd.tile_rows(16384, 17408, 5120) == 256
    assert bd.tile_rows(32768, 5120, 5120) == 256
    assert bd.tile_rows(2054, 5120, 5120) == 192       # mixed batch: 180 tiles of 256 rows, 220 of 192
    assert bd.tile_rows(2054, 17408, 5120) == 192
    assert bd.tile_rows(700, 17408, 136) == 256        # 204 tiles; 192 or 128 rows would take two waves
    assert bd.tile_rows(700, 11008, 136) == 192
    assert bd.tile_rows(300, 1000, 136) == 128
    assert bd.tile_rows(129, 5120, 5120) == 128
    assert bd.tile_rows(128, 5120, 5120) == 0          # decode path
    assert bd.tile_rows(300, 1000, 136, "f32") == 0    # test mode
    assert bd.tile_rows(300, 1000, 252) == 0           # invalid K


def call(**kw):
    a = dict(X=FAKE, seg_starts=[0, 32, 64], seg_adapter=[-1, 0], W=FAKE2, A=[FAKE3], B=[FAKE4], rank=16,
             scale=0.5, Y=FAKE5, M=64, N=512, K=256, dtype="bf16", workspace=FAKE * 320,
             workspace_bytes_=1 << 24, stream=None)
    a.update(kw)
    return bd.lora_proj_raw(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(X=None), bd.LORA_EINVAL),
    (dict(W=None), bd.LORA_EINVAL),
    (dict(Y=None), bd.LORA_EINVAL),
    (dict(X=FAKE + 8), bd.LORA_EINVAL),                                  # misaligned
    (dict(N=0), bd.LORA_EINVAL),
    (dict(K=0), bd.LORA_EINVAL),
    (dict(M=-1), bd.LORA_EINVAL),
    (dict(K=250), bd.LORA_EUNSUPPORTED),                                 # K % 8
    (dict(dtype=7), bd.LORA_EUNSUPPORTED),
    (dict(rank=24), bd.LORA_EUNSUPPORTED),                               # rank % 16
    (dict(rank=528), bd.LORA_EUNSUPPORTED),
    (dict(rank=0), bd.LORA_EUNSUPPORTED),
    (dict(M=1 << 20, K=1 << 12, seg_starts=[0, 1 << 20], seg_adapter=[-1]), bd.LORA_EUNSUPPORTED),  # X >= 2 GiB
    (dict(seg_starts=[1, 32, 64]), bd.LORA_ESEGMENTS),
    (dict(seg_starts=[0, 32, 63]), bd.LORA_ESEGMENTS),
    (dict(seg_starts=[0, 40, 32, 64], seg_adapter=[-1, 0, 0]), bd.LORA_ESEGMENTS),
    (dict(seg_starts=[0], seg_adapter=[]), bd.LORA_ESEGMENTS),            # M > 0 with no segment
    (dict(seg_adapter=[-1, 1]), bd.LORA_EADAPTER),
    (dict(seg_adapter=[-2, 0]), bd.LORA_EADAPTER),
    (dict(A=[None]), bd.LORA_EADAPTER),
    (dict(B=[None]), bd.LORA_EADAPTER),
    (dict(A=[FAKE3 + 4]), bd.LORA_EINVAL),
    (dict(workspace=None, workspace_bytes_=0), bd.LORA_EWORKSPACE),
    (dict(workspace_bytes_=64 * 16 * 4), bd.LORA_EWORKSPACE),            # below the decode partials
    (dict(M=300, seg_starts=[0, 32, 300], workspace_bytes_=300 * 16 * 4 - 1), bd.LORA_EWORKSPACE),
    (dict(Y=FAKE + 4096), bd.LORA_EINVAL),                               # Y overlaps X
    (dict(Y=FAKE2 + 4096), bd.LORA_EINVAL),                              # Y overlaps W
    (dict(Y=FAKE3), bd.LORA_EINVAL),                                     # Y overlaps A
    (dict(workspace=FAKE5 + 16), bd.LORA_EINVAL),                        # workspace inside Y
])
def test_rejected_before_launch(kw, code):
    assert call(**kw) == code


def test_segment_and_adapter_limits():
    n = bd.MAX_SEGMENTS + 1
    starts = list(range(n + 1))
    alternating = [i % 2 - 1 for i in range(n)]               # -1, 0, -1, 0, ... never merges
    assert call(M=n, seg_starts=starts, seg_adapter=alternating) == bd.LORA_EUNSUPPORTED
    too_many = [FAKE3] * (bd.MAX_ADAPTERS + 1)
    assert call(A=too_many, B=[FAKE4] * (bd.MAX_ADAPTERS + 1)) == bd.LORA_EUNSUPPORTED


def test_empty_batch_is_a_no_op():
    # M == 0 returns OK without touching the GPU, whatever the pointers.
    assert call(M=0, seg_starts=[0], seg_adapter=[], X=None, Y=None) == bd.LORA_OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(bd, "_lib", None)
    monkeypatch.setattr(bd, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="missing"):
        bd.load()


def test_per_adapter_scales_rejected_before_launch():
    # the per-adapter entry point shares the single-scale call's checks
    assert call(scale=[0.5], seg_starts=[1, 32, 64]) == bd.LORA_ESEGMENTS
    assert call(scale=[0.5], A=[None]) == bd.LORA_EADAPTER
    assert call(scale=[0.5], rank=24) == bd.LORA_EUNSUPPORTED
    assert call(scale=[0.5], M=0, seg_starts=[0], seg_adapter=[], X=None, Y=None) == bd.LORA_OK
    with pytest.raises(ValueError):
        call(scale=[0.5, 1.0])                                   # one scale per adapter
    # NULL scales with adapters present is an invalid argument
    lib = bd.load()
    starts = (ctypes.c_int32 * 3)(0, 32, 64)
    adapt = (ctypes.c_int32 * 2)(-1, 0)
    a_arr = (ctypes.c_void_p * 1)(FAKE3)
    b_arr = (ctypes.c_void_p * 1)(FAKE4)
    st = lib.lora_proj_multi(FAKE, starts, adapt, 2, FAKE2, a_arr, b_arr, 1, 16, None, FAKE5,
                             64, 512, 256, bd.DTYPES["bf16"], FAKE * 320, 1 << 24, None)
    assert st == bd.LORA_EINVAL


@pytest.mark.parametrize("kw,code", [
    (dict(slices=[256, 512]), bd.LORA_EINVAL),                  # widths do not sum to N = 512
    (dict(slices=[0, 512]), bd.LORA_EINVAL),                    # empty slice
    (dict(slices=[128, 384]), bd.LORA_EUNSUPPORTED),            # not a multiple of 256
    (dict(slices=[256] * 5, N=1280), bd.LORA_EUNSUPPORTED),     # more than 4 slices
    (dict(slices=[511]), bd.LORA_EINVAL),                       # one slice must be N wide
    # the stacked A is 2 r rows: the plain call's workspace is too small for the sliced T
    (dict(slices=[256, 256], M=300, seg_starts=[0, 32, 300],
          workspace_bytes_=bd.WORKSPACE_COUNTER_BYTES + 300 * 16 * 4), bd.LORA_EWORKSPACE),
])
def test_sliced_rejected_before_launch(kw, code):
    assert call(**kw) == code


def test_sliced_workspace_query():
    C = bd.WORKSPACE_COUNTER_BYTES
    assert bd.workspace_bytes(16384, 15360, 5120, 256, 1, "bf16", 3) == C + 16384 * 768 * 4
    assert bd.workspace_bytes(300, 512, 256, 16, 1, "bf16", 1) == bd.workspace_bytes(300, 512, 256, 16, 1)
    dec1 = bd.workspace_bytes(70, 15360, 5120, 256, 1)
    dec3 = bd.workspace_bytes(70, 15360, 5120, 256, 1, "bf16", 3)
    assert dec3 > dec1 and dec3 % 256 == 0
    assert bd.workspace_bytes(70, 15360, 5120, 256, 1, "bf16", 5) == 0       # too many slices
    assert bd.workspace_bytes(70, 15000, 5120, 256, 1, "bf16", 3) == 0       # N not slice-aligned


def ranked_call(**kw):
    a = dict(X=FAKE, seg_starts=[0, 32, 48, 64], seg_adapter=[-1, 0, 1], W=FAKE2, A=[FAKE3, FAKE3 + (1 << 22)],
             B=[FAKE4, FAKE4 + (1 << 22)], ranks=[16, 48], scales=[0.5, 1.0], Y=FAKE5, M=64, N=512, K=256,
             dtype="bf16", workspace=FAKE * 320, workspace_bytes_=1 << 24, stream=None)
    a.update(kw)
    return bd.lora_proj_ranked_raw(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(ranks=[16, 24]), bd.LORA_EUNSUPPORTED),               # a rank not a multiple of 16
    (dict(ranks=[528, 16]), bd.LORA_EUNSUPPORTED),              # above the largest rank
    (dict(ranks=[0, 48]), bd.LORA_EUNSUPPORTED),                # a named adapter with no rank
    (dict(ranks=[16, 48], seg_adapter=[-1, 0, 2]), bd.LORA_EADAPTER),
    (dict(A=[FAKE3, None]), bd.LORA_EADAPTER),
    (dict(Y=FAKE3 + (1 << 22) + 4096), bd.LORA_EINVAL),          # Y overlaps the rank-48 adapter's A
    # the workspace of the largest rank (48) is needed: one sized for rank 16 is too small
    (dict(M=300, seg_starts=[0, 32, 48, 300], workspace_bytes_=bd.workspace_bytes(300, 512, 256, 16, 2)),
     bd.LORA_EWORKSPACE),
])
def test_ranked_rejected_before_launch(kw, code):
    assert ranked_call(**kw) == code


def test_ranked_checks():
    # an empty batch is a no-op whatever the ranks
    assert ranked_call(ranks=[16, 7], seg_adapter=[-1, 0, 0], M=0, seg_starts=[0, 0, 0, 0], X=None,
                       Y=None) == bd.LORA_OK
    with pytest.raises(ValueError):
        ranked_call(ranks=[16])                                  # one rank per adapter
    lib = bd.load()
    starts = (ctypes.c_int32 * 3)(0, 32, 64)
    adapt = (ctypes.c_int32 * 2)(-1, 0)
    a_arr = (ctypes.c_void_p * 1)(FAKE3)
    b_arr = (ctypes.c_void_p * 1)(FAKE4)
    widths = (ctypes.c_int64 * 1)(512)
    scales = (ctypes.c_float * 1)(0.5)
    ranks = (ctypes.c_int32 * 1)(16)
    # NULL ranks or NULL scales with adapters present
    for r, sc in ((None, scales), (ranks, None)):
        st = lib.lora_proj_ranked(FAKE, starts, adapt, 2, FAKE2, a_arr, b_arr, 1, r, sc, 1, widths, FAKE5,
                                  64, 512, 256, bd.DTYPES["bf16"], FAKE * 320, 1 << 24, None)
        assert st == bd.LORA_EINVAL


def q4_call(**kw):
    a = dict(X=FAKE, seg_starts=[0, 32, 64], seg_adapter=[-1, 0], Wq=FAKE2, Wp=FAKE2 + (1 << 19), A=[FAKE3],
             B=[FAKE4], rank=16, scales=[0.5], Y=FAKE5, M=64, N=512, K=256, dtype="bf16", workspace=FAKE * 320,
             workspace_bytes_=1 << 24, stream=None)
    a.update(kw)
    return bd.lora_proj_q4_raw(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(Wp=None), bd.LORA_EINVAL),
    (dict(dtype="f32"), bd.LORA_EUNSUPPORTED),       # no fp32 test mode for 4-bit weights
    (dict(K=192), bd.LORA_EUNSUPPORTED),             # K not a multiple of the 128-wide group
    (dict(Wp=FAKE2 + 8), bd.LORA_EINVAL),            # misaligned params
    (dict(Y=FAKE2 + 4096), bd.LORA_EINVAL),          # Y overlaps the codes
    (dict(M=300, seg_starts=[0, 32, 300], workspace_bytes_=bd.WORKSPACE_COUNTER_BYTES + 300 * 16 * 4),
     bd.LORA_EWORKSPACE),                            # the prefill path also needs the bf16 copy of W
])
def test_q4_rejected_before_launch(kw, code):
    assert q4_call(**kw) == code


def test_q4_workspace_query():
    C = bd.WORKSPACE_COUNTER_BYTES
    assert bd.q4_workspace_bytes(16384, 5120, 5120, 256) == C + 16384 * 256 * 4 + 5120 * 5120 * 2
    assert bd.q4_workspace_bytes(16384, 5120, 5120, 256, 0) == C + 5120 * 5120 * 2
    assert bd.q4_workspace_bytes(70, 5120, 5120, 256) == bd.workspace_bytes(70, 5120, 5120, 256)
    assert bd.q4_workspace_bytes(70, 5120, 5000, 256) == 0
    assert bd.q4_workspace_bytes(70, 5120, 5120, 256, 1, "f32") == 0


@pytest.mark.parametrize("kw,code", [
    (dict(l=47), bd.LORA_EUNSUPPORTED),                 # odd l
    (dict(rank=64), bd.LORA_EUNSUPPORTED),              # rank > l
    (dict(l=514, rank=16), bd.LORA_EUNSUPPORTED),       # l > 512
    (dict(power_iters=9), bd.LORA_EUNSUPPORTED),
    (dict(Wa=None), bd.LORA_EINVAL),
    (dict(B=FAKE5 + 4), bd.LORA_EINVAL),                # misaligned
    (dict(workspace_bytes_=1024), bd.LORA_EWORKSPACE),
    (dict(B=FAKE), bd.LORA_EINVAL),                     # B overlaps W_adapted
])
def test_extract_rejected_before_launch(kw, code):
    a = dict(Wa=FAKE, Wb=FAKE2, N=256, K=512, omega=FAKE3, l=48, rank=32, power_iters=2, B=FAKE5,
             A=FAKE5 + (1 << 20), sigma=FAKE5 + (2 << 20), workspace=FAKE * 512, workspace_bytes_=1 << 26)
    a.update(kw)
    assert bd.extract_raw(a["Wa"], a["Wb"], a["N"], a["K"], a["omega"], a["l"], a["rank"], a["power_iters"],
                          a["B"], a["A"], a["sigma"], a["workspace"], a["workspace_bytes_"]) == code


def test_extract_workspace_query():
    assert bd.extract_workspace_bytes(5120, 5120, 272, 256) > 5120 * 5120 * 4
    assert bd.extract_workspace_bytes(5120, 5120, 271, 256) == 0


def test_probes_reject_bad_arguments():
    """The measurement probes check their arguments on the host before any launch."""
    st, _ = bd.probe_mfma_bf16_raw(0, FAKE)
    assert st == bd.LORA_EINVAL
    st, _ = bd.probe_mfma_bf16_raw(1 << 25, FAKE)
    assert st == bd.LORA_EINVAL
    st, _ = bd.probe_mfma_bf16_raw(10, None)
    assert st == bd.LORA_EINVAL
    assert bd.probe_read_raw(FAKE, 0, FAKE2) == bd.LORA_EINVAL
    assert bd.probe_read_raw(FAKE, 24, FAKE2) == bd.LORA_EINVAL          # not a multiple of 16
    assert bd.probe_read_raw(FAKE + 8, 32, FAKE2) == bd.LORA_EINVAL      # unaligned
    assert bd.probe_read_raw(None, 32, FAKE2) == bd.LORA_EINVAL
    assert bd.probe_read_raw(FAKE, 32, None) == bd.LORA_EINVAL


def test_binding_rejects_host_tensors_and_wrong_shapes():
    """The binding hands the library pointers and sizes only, so it refuses operands that are not
    device tensors, or whose shapes disagree with the call's, before anything reaches the device."""
    torch = pytest.importorskip("torch")
    dev = torch.device("cuda", 0)
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError, match="CUDA"):
        bd._check_operands(dev, {"omega": x})
    with pytest.raises(ValueError, match="shape"):
        bd._check_operands(dev, {}, [("W_base", x, (4, 16))])
    bd._check_operands(dev, {"workspace": None}, [("W", x, (4, 8))])


def test_wrapper_refuses_raw_stream_handle():
    """The tensor wrappers allocate on the stream they enqueue on, so they take torch streams only;
    a raw handle is refused before anything reaches the device."""
    import pytest
    import torch
    with pytest.raises(TypeError):
        bd._stream_of(12345, torch.device("cuda:0"))
