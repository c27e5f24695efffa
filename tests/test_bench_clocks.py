"""bench.py's clock sampler on the host: the current DPM level is the line marked '*' of the
driver's pp_dpm_sclk / pp_dpm_mclk files; a summary holds median, min and max over the samples."""
from __future__ import annotations

import os
import sys
import time

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


def test_reads_the_marked_level(tmp_path):
    c = bench.ClockSampler()
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("S: 1550Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    assert c._read(str(f)) == 1550
    f.write_text("0: 500Mhz\n1: 2400Mhz *\n")
    assert c._read(str(f)) == 2400
    f.write_text("0: 500Mhz\n1: 2400Mhz\n")
    assert c._read(str(f)) is None
    assert c._read(str(tmp_path / "missing")) is None


def test_samples_while_running(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("S: 1600Mhz *\n")
    c = bench.ClockSampler(period_s=0.001)
    c.files = {"sclk": str(f)}
    c.samples = {"sclk": []}
    with c:
        time.sleep(0.05)
    s = c.summary()
    assert s["sclk_mhz"]["median"] == s["sclk_mhz"]["min"] == s["sclk_mhz"]["max"] == 1600
    assert s["sclk_mhz"]["samples"] >= 2


def test_no_files_no_summary():
    c = bench.ClockSampler()
    c.files, c.samples = {}, {}
    with c:
        pass
    assert c.summary() is None
