"""The measurement probes (lora_probe.h) through the C-ABI: they launch, and the rates they imply sit
between a floor and the published peaks (2.5 PFLOP/s dense bf16 MFMA, 8 TB/s HBM), so a miscounted
flop or byte figure would show."""
from __future__ import annotations

import pytest

from gpu_util import log
from rank_adapted_gemm_amd import binding as bd

pytestmark = pytest.mark.gpu


def _time(fn):
    import torch
    st = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    fn()
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e-3


def test_mfma_probe_rate():
    import torch
    sink = torch.zeros(1024, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    out = {}

    def run():
        st, flop = bd.probe_mfma_bf16_raw(400, sink.data_ptr(), stream)
        assert st == bd.LORA_OK
        out["flop"] = flop
    t = _time(run)
    tflops = out["flop"] / t / 1e12
    log(f"mfma probe: {tflops:.0f} TFLOP/s")
    assert 100 < tflops < 2517


def test_read_probe_rate():
    import torch
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")   # 16x the MALL: read from HBM
    sink = torch.zeros(1024, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def run():
        for _ in range(4):
            assert bd.probe_read_raw(buf.data_ptr(), buf.numel(), sink.data_ptr(), stream) == bd.LORA_OK
    gbs = 4 * buf.numel() / _time(run) / 1e9
    log(f"read probe: {gbs:.0f} GB/s")
    assert 500 < gbs < 8000
