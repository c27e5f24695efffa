#!/usr/bin/env python3
"""Throughput of the mixed-adapter LoRA projection on one MI355X.

One step is one pass of the whole hot path — segment scheduling, shrink,
fused base product + expand, bf16 store — over every projection of the
workload, with all inputs already resident in HBM:

  prefill16k (the headline): one adapted layer, 16,384 token rows that all
      name the adapter, seven projections (q, k, v, o 5120->5120; gate, up
      5120->17408; down 17408->5120), rank 256.  Reported in TFLOP/s and as a
      fraction of the bf16 MFMA peak.
  suffix (decode line): 24 adapted layers x 7 projections, 64 adapter rows plus
      6 base-only decode rows (M = 70).  Reported in GB/s and as a fraction of
      HBM bandwidth, twice: one call per projection, and grouped (q/k/v as one
      sliced call and gate/up as another, the way a server stores those
      groups; o and down alone), 4 calls per layer over the same weights.

Algorithmic work per call: FLOP = 2 M N K + 2 M_a r (K + N); bytes = W + X + Y,
plus A_a and B_a when the call has adapter rows (bf16).

The output kernel (base product + expand + store) is timed on its own with HIP
events recorded around every launch inside the timed region; its achieved rate
is the roofline figure.  The CPU baseline times the fp64 oracle on a bounded
sample of rows of the same workload.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import contextlib
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from rank_adapted_gemm_amd import binding as bd  # noqa: E402
from rank_adapted_gemm_amd import synth  # noqa: E402

METRIC = "TFLOP/s + %MFMA peak (16k prefill); GB/s + %HBM peak (decode batch)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "rank_adapted_gemm_amd", "csrc", "lora_bf16.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ HIP events
class HipEvents:
    """hipEvent_t pairs through the HIP runtime (the output kernel is timed on its own stream).

    The events only time: they are created without the system-scope fence (a cache writeback and
    invalidate) that a default event performs when it is recorded.  Each record still leaves the
    GPU idle for a few microseconds before the next launch.  The step's wall clock ends with a
    full device synchronization."""

    DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence

    def __init__(self):
        self.lib = bd.load()      # resolves to the process's one HIP runtime (torch's)
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def pair(self):
        a, b = ctypes.c_void_p(), ctypes.c_void_p()
        for e in (a, b):
            if self.lib.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.events.append(e)
        return a.value, b.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for e in self.events:
            self.lib.hipEventDestroy(e)
        self.events = []


# ------------------------------------------------------------------ clocks
class ClockSampler:
    """The GPU's current shader and memory clock levels, sampled every few milliseconds from a
    thread while a timed region runs (the level marked '*' in the driver's pp_dpm_sclk and
    pp_dpm_mclk files).  The driver reports DPM levels; the effective clock under load comes from
    the counter profiles.  Where the files are missing, the summary is None."""

    def __init__(self, period_s=0.004):
        import glob
        self.files = {}
        for key in ("sclk", "mclk"):
            paths = sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{key}"))
            if paths:
                self.files[key] = paths[0]
        self.period = period_s
        self.samples = {k: [] for k in self.files}
        self._stop = None
        self._thread = None

    def _read(self, path):
        try:
            for line in open(path):
                if line.rstrip().endswith("*"):
                    return int(line.split(":", 1)[1].strip().split("M")[0])
        except (OSError, ValueError, IndexError):
            pass
        return None

    def _run(self):
        while not self._stop.is_set():
            for k, path in self.files.items():
                v = self._read(path)
                if v is not None:
                    self.samples[k].append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        import threading
        if self.files:
            self._stop = threading.Event()
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        out = {}
        for k, v in self.samples.items():
            if v:
                out[f"{k}_mhz"] = dict(median=int(np.median(v)), min=int(min(v)), max=int(max(v)), samples=len(v))
        return out or None


# ------------------------------------------------------------------ work model
def adapter_rows(seg_starts, seg_adapter):
    s = np.asarray(seg_starts)
    return int(sum(s[g + 1] - s[g] for g in range(len(seg_adapter)) if seg_adapter[g] >= 0))


def call_work(M, Ma, N, K, r, S=1, q4=False):
    """(main-kernel flops, shrink flops, algorithmic bytes) of one call of S slices.

    With 4-bit base weights W counts as its codes (N K / 2 bytes) plus one 4-byte params word per
    128-wide group."""
    main = 2 * M * N * K + 2 * Ma * N * r
    shrink = 2 * Ma * S * r * K
    w_bytes = N * K // 2 + N * (K // 128) * 4 if q4 else 2 * N * K
    byts = w_bytes + 2 * (M * K + M * N + ((S * r * K + N * r) if Ma else 0))
    return main, shrink, byts


# ------------------------------------------------------------------ device workloads
def device_layer(cfg, layer, M, dev, shapes=synth.PROJECTIONS):
    """Inputs of one adapted layer drawn on the device (same shapes and sigmas as the host recipe)."""
    widths = sorted({K for _, K, _ in shapes})
    xs = {K: synth.device_normal_bf16((M, K), 1.0, synth.seed_of(cfg, layer, proj, synth.T_X), dev)
          for K, proj in zip(widths, (synth.X_NARROW, synth.X_WIDE))}
    projs = []
    for pi, (name, K, N) in enumerate(shapes):
        W = synth.device_normal_bf16((N, K), synth.SIGMA_WAB, synth.seed_of(cfg, layer, pi, synth.T_W), dev)
        A = synth.device_normal_bf16((synth.RANK, K), synth.SIGMA_WAB, synth.seed_of(cfg, layer, pi, synth.T_A), dev)
        B = synth.device_normal_bf16((N, synth.RANK), synth.SIGMA_WAB, synth.seed_of(cfg, layer, pi, synth.T_B), dev)
        projs.append(dict(name=name, K=K, N=N, X=xs[K], W=W, A=A, B=B))
    return projs


def group_layer(projs):
    """The layer's q/k/v and gate/up as sliced calls (weights concatenated along N, A stacked)."""
    import torch
    by = {p["name"]: p for p in projs}

    def group(name, members):
        ps = [by[m] for m in members]
        g = dict(name=name, K=ps[0]["K"], N=sum(p["N"] for p in ps), X=ps[0]["X"],
                 W=torch.cat([p["W"] for p in ps]), A=torch.cat([p["A"] for p in ps]),
                 B=torch.cat([p["B"] for p in ps]), slices=[p["N"] for p in ps])
        for p in ps:
            del p["W"], p["A"], p["B"]
        return g
    return [group("qkv", ("q", "k", "v")), by["o"], group("gate_up", ("gate", "up")), by["down"]]


class StepRunner:
    """All calls of one step over preallocated outputs and one shared workspace."""

    def __init__(self, layers, seg_starts, seg_adapter, scale, dev):
        import torch
        self.calls = []
        M = layers[0][0]["X"].shape[0]
        self.M, self.Ma = M, adapter_rows(seg_starts, seg_adapter)
        self.seg_starts, self.seg_adapter, self.scale = list(seg_starts), list(seg_adapter), scale
        nad = max(len(p["A"]) if isinstance(p["A"], list) else 1 for p in layers[0])
        ws = max(bd.q4_workspace_bytes(M, p["N"], p["K"], synth.RANK, nad, "bf16", len(p.get("slices", [0])))
                 if "Wq" in p else
                 bd.workspace_bytes(M, p["N"], p["K"], synth.RANK, nad, "bf16", len(p.get("slices", [0])))
                 for p in layers[0])
        self.workspace = torch.zeros(ws, dtype=torch.uint8, device=dev)   # counter area starts at zero
        self.outs = {}
        for projs in layers:
            for p in projs:
                key = (p["N"],)
                if key not in self.outs:     # outputs of equal shape are reused across layers
                    self.outs[key] = torch.empty((M, p["N"]), dtype=torch.bfloat16, device=dev)
                self.calls.append(p)
        self.stream = torch.cuda.current_stream(dev).cuda_stream

    def work(self):
        main = shrink = byts = 0
        for p in self.calls:
            a, b, c = call_work(self.M, self.Ma, p["N"], p["K"], synth.RANK, len(p.get("slices", [0])), "Wq" in p)
            main, shrink, byts = main + a, shrink + b, byts + c
        return main, shrink, byts

    def step(self, events=None):
        ws = self.workspace
        for i, p in enumerate(self.calls):
            if "Wq" in p:
                st = bd.lora_proj_q4_raw(p["X"].data_ptr(), self.seg_starts, self.seg_adapter, p["Wq"].data_ptr(),
                                         p["Wp"].data_ptr(), [p["A"].data_ptr()], [p["B"].data_ptr()], synth.RANK,
                                         self.scale, self.outs[(p["N"],)].data_ptr(), self.M, p["N"], p["K"], "bf16",
                                         ws.data_ptr(), ws.numel(), self.stream, p.get("slices"))
                if st != bd.LORA_OK:
                    raise bd.LoraError(st, bd.status_string(st))
                continue
            As, Bs = (p["A"], p["B"]) if isinstance(p["A"], list) else ([p["A"]], [p["B"]])
            st = bd.lora_proj_raw(p["X"].data_ptr(), self.seg_starts, self.seg_adapter, p["W"].data_ptr(),
                                  [t.data_ptr() for t in As], [t.data_ptr() for t in Bs], synth.RANK, self.scale,
                                  self.outs[(p["N"],)].data_ptr(), self.M, p["N"], p["K"], "bf16",
                                  ws.data_ptr(), ws.numel(), self.stream,
                                  None if events is None else events[i], p.get("slices"))
            if st != bd.LORA_OK:
                raise bd.LoraError(st, bd.status_string(st))


def time_steps(runner, steps, warmup, hip, events=True, clocks=None):
    """Wall time of `steps` steps; with `events`, also each output kernel's duration.

    The decode stack is timed without events: a record costs a little time even without
    its system fence, which matters next to a ~10 us decode call.
    """
    import torch
    for _ in range(warmup):
        runner.step()
    torch.cuda.synchronize()
    pairs = [[hip.pair() for _ in runner.calls] for _ in range(steps)] if events else [None] * steps
    torch.cuda.synchronize()
    with clocks if clocks is not None else contextlib.nullcontext():   # clock samples over the timed steps
        t0 = time.perf_counter()
        for s in range(steps):
            runner.step(events=pairs[s])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    if not events:
        return wall, None
    main_ms = [[hip.elapsed_ms(a, b) for (a, b) in row] for row in pairs]
    return wall, np.array(main_ms)


# ------------------------------------------------------------------ CPU baseline
def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _host_layer(cfg, M):
    """Host-recipe inputs of a workload's layer 0: {K: X values} and [(name, K, N, W, A, B)]."""
    xs = {K: synth.layer_input(cfg, 0, M, K)[1] for K in sorted({K for _, K, _ in synth.PROJECTIONS})}
    projs = []
    for pi, (name, K, N) in enumerate(synth.PROJECTIONS):
        (_, Wf), (_, Af), (_, Bf) = synth.projection_weights(cfg, 0, pi, K, N)
        projs.append((name, K, N, Wf, Af, Bf))
    return xs, projs


def cpu_baseline(rows: int):
    """The fp64 oracle as it stands, on the host cores, beside the GPU lines:

      * prefill16k: `rows` token rows of each of the 7 projections (16,384 = the whole workload),
        on every BLAS thread (the `value`), and 256 rows per projection on one thread;
      * mixed (2,054 rows, 7 projections) in full;
      * suffix (M = 70): layer 0's 7 projections in full, scaled by 24 for the stack (every layer
        has the same shapes, so the same cost).
    """
    from oracle import lora_proj_ref
    import threadpoolctl
    threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1

    def time_layer(xs, projs, starts, labels, M, Ma):
        total, flops = 0.0, 0
        for name, K, N, Wf, Af, Bf in projs:
            X = xs[K]
            t0 = time.perf_counter()
            lora_proj_ref(X, starts, labels, Wf, [Af], [Bf], 1.0)
            total += time.perf_counter() - t0
            main, shrink, _ = call_work(M, Ma, N, K, synth.RANK)
            flops += main + shrink
        return total, flops

    g = np.random.Generator(np.random.PCG64(7))
    _, projs2 = _host_layer(2, 1)   # weights of the prefill16k layer (X drawn below per sample)
    # all threads, prefill16k rows
    xs = {K: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(g.standard_normal((rows, K), dtype=np.float32)))
          for K in (5120, 17408)}
    t_all, f_all = time_layer(xs, projs2, [0, rows], [0], rows, rows)
    log(f"  cpu oracle prefill16k: {rows} rows x 7 projections, {f_all / 1e9:.0f} GFLOP in {t_all:.1f} s "
        f"on {threads} threads")
    # one thread, 256 rows
    r1 = 256
    xs1 = {K: v[:r1] for K, v in xs.items()}
    with threadpoolctl.threadpool_limits(1):
        t_one, f_one = time_layer(xs1, projs2, [0, r1], [0], r1, r1)
    log(f"  cpu oracle prefill16k, one thread: {r1} rows x 7, {f_one / 1e9:.0f} GFLOP in {t_one:.1f} s")
    del xs, xs1, projs2
    # mixed and suffix in full
    out = {}
    for name in ("mixed", "suffix"):
        w = synth.WORKLOADS[name]
        xs, projs = _host_layer(w["cfg"], w["M"])
        ma = adapter_rows(w["seg_starts"], w["seg_adapter"])
        t, f = time_layer(xs, projs, list(w["seg_starts"]), list(w["seg_adapter"]), w["M"], ma)
        byts = sum(call_work(w["M"], ma, N, K, synth.RANK)[2] for _, K, N, *_ in projs)
        layers = w["layers"]
        out[name] = dict(seconds_per_step=round(t * layers, 3), layers_timed=1, layers_per_step=layers,
                         tflops=round(f / t / 1e12, 4), gbs=round(byts / t / 1e9, 2))
        log(f"  cpu oracle {name}: 7 projections in full, {t:.2f} s per layer ({layers} per step)")
        del xs, projs
    return dict(value=f_all / t_all / 1e12, unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample=f"{rows} of 16384 rows of each of the 7 prefill16k projections, fp64 numpy oracle; "
                       f"{f_all / 1e9:.1f} GFLOP in {t_all:.1f} s",
                cpu_model=_cpu_model(), nproc=int(os.cpu_count() or 1), affinity_cpus=int(affinity),
                blas_threads=int(threads),
                one_thread=dict(value=round(f_one / t_one / 1e12, 5), unit="TFLOP/s",
                                sample=f"{r1} rows of each of the 7 prefill16k projections on one thread"),
                mixed_full=dict(out["mixed"], sample="all 2,054 rows of the mixed batch's 7 projections"),
                suffix_full=dict(out["suffix"], sample="all 70 rows of the suffix batch's 7 projections of "
                                                       "layer 0; 24 layers of the same shapes per step"))


def traffic_record():
    """HBM bytes per output-kernel launch from the committed rocprofv3 counter runs, if current."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
        src = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
        if rec.get("kernel_source_sha256") == src:
            return rec.get("bytes_per_launch")
    except (OSError, ValueError):
        pass
    return None



# ------------------------------------------------------------------ the two timed workloads
def run_prefill(a, dev, hip, name="prefill16k", steps=None, warmup=None):
    import torch
    w = synth.WORKLOADS[name]
    steps = a.steps if steps is None else steps
    warmup = a.warmup if warmup is None else warmup
    log(f"{name}: drawing {w['layers']} layer(s) on the device")
    layers = [device_layer(w["cfg"], l, w["M"], dev, synth.projections(name)) for l in range(w["layers"])]
    runner = StepRunner(layers, w["seg_starts"], w["seg_adapter"], w["scale"], dev)
    main_flops, shrink_flops, byts = runner.work()
    log(f"{name}: {warmup} warmup + {steps} timed steps of {len(runner.calls)} calls")
    clocks = ClockSampler()
    wall, main_ms = time_steps(runner, steps, warmup, hip, clocks=clocks)
    ms_per_step = wall * 1e3 / steps
    step_flops = main_flops + shrink_flops
    value = step_flops / (ms_per_step / 1e3) / 1e12
    main_achieved = main_flops * steps / (main_ms.sum() / 1e3) / 1e12
    n7 = len(synth.projections(name))
    per_proj_ms = main_ms.reshape(steps, -1, n7).mean(axis=(0, 1))   # per projection, over layers and steps
    by_proj = main_ms.reshape(steps, -1, n7).transpose(2, 0, 1).reshape(n7, -1)
    log(f"{name}: {ms_per_step:.3f} ms/step, {value:.1f} TFLOP/s; output kernel {main_achieved:.1f} TFLOP/s; "
        + ", ".join(f"{p['name']} {t:.3f}" for p, t in zip(runner.calls, per_proj_ms)))
    roofline = dict(bound="mfma", achieved=round(main_achieved, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(main_achieved / PEAK_BF16_TFLOPS, 4), traffic=traffic_record(),
                    kernel="main_kernel<Tile<256,256,2,2>, bf16 out>",
                    launch_avg_ms=round(float(main_ms.mean()), 4),
                    launch_median_ms=round(float(np.median(main_ms)), 4), launch_min_ms=round(float(main_ms.min()), 4),
                    per_projection_ms={p["name"]: round(float(t), 4) for p, t in zip(runner.calls, per_proj_ms)},
                    per_projection_median_ms={p["name"]: round(float(np.median(d)), 4)
                                              for p, d in zip(runner.calls, by_proj)},
                    per_projection_min_ms={p["name"]: round(float(d.min()), 4) for p, d in zip(runner.calls, by_proj)},
                    clocks=clocks.summary())
    n_calls = len(runner.calls)
    del runner, layers
    torch.cuda.empty_cache()
    return dict(value=value, ms_per_step=ms_per_step, flops=step_flops, bytes=byts, roofline=roofline,
                calls=n_calls, steps=steps)


MIXED_ADAPTERS = synth.MIXED_ADAPTERS


def run_prefill_mixed(a, dev, hip):
    """prefill16k's layer with four adapters per projection in a batch of short interleaved segments
    (the many-adapters case): TFLOP/s of the algorithmic work, whose adapter rows are those naming any."""
    import torch
    w = synth.WORKLOADS["prefill16k"]
    M = w["M"]
    layer = device_layer(w["cfg"], 0, M, dev)
    for pi, p in enumerate(layer):   # adapters 1..3 of each projection, drawn like adapter 0
        p["A"] = [p["A"]] + [synth.device_normal_bf16((synth.RANK, p["K"]), synth.SIGMA_WAB,
                                                      synth.extra_adapter_seed(w["cfg"], 0, pi, synth.T_A, j), dev)
                             for j in range(1, MIXED_ADAPTERS)]
        p["B"] = [p["B"]] + [synth.device_normal_bf16((p["N"], synth.RANK), synth.SIGMA_WAB,
                                                      synth.extra_adapter_seed(w["cfg"], 0, pi, synth.T_B, j), dev)
                             for j in range(1, MIXED_ADAPTERS)]
    starts, labels = synth.mixed_table(M, MIXED_ADAPTERS)
    runner = StepRunner([layer], starts, labels, 1.0, dev)
    main_flops, shrink_flops, _ = runner.work()
    wall, main_ms = time_steps(runner, a.steps, a.warmup, hip)
    ms_per_step = wall * 1e3 / a.steps
    value = (main_flops + shrink_flops) / (ms_per_step / 1e3) / 1e12
    main_achieved = main_flops * a.steps / (main_ms.sum() / 1e3) / 1e12
    ma = runner.Ma
    log(f"prefill16k_mixed: {len(labels)} segments, {ma} adapter rows: {ms_per_step:.3f} ms/step, "
        f"{value:.1f} TFLOP/s; output kernel {main_achieved:.1f} TFLOP/s")
    del runner, layer
    torch.cuda.empty_cache()
    return dict(workload=f"prefill16k layer with {MIXED_ADAPTERS} adapters per projection; {M} rows in "
                         f"{len(labels)} segments of 20-140 rows, each naming one adapter or none (seeded)",
                value=round(value, 2), unit="TFLOP/s", ms_per_step=round(ms_per_step, 4),
                frac=round(value / PEAK_BF16_TFLOPS, 4), main_kernel_tflops=round(main_achieved, 2),
                adapter_rows=ma)


RANKED_RANKS = (64, 128, 192, 256)


def run_ranked(a, dev):
    """Adapters of different ranks in one batch: four adapters of ranks 64, 128, 192 and 256 per
    projection over one layer, served with compact factors (lora_proj_ranked) and, for comparison,
    zero-padded to rank 256 (lora_proj_multi); prefill16k's 212-segment table and a 70-row decode
    batch (4 x 16 adapter rows, 6 base rows).  ms per step of 7 calls, each variant timed alone."""
    import torch
    out = {}
    for path, wname, M in (("prefill", "prefill16k", 16384), ("decode", "suffix", 70)):
        cfg = synth.WORKLOADS[wname]["cfg"]
        layer = device_layer(cfg, 0, M, dev)
        if path == "prefill":
            starts, labels = synth.mixed_table(M, len(RANKED_RANKS))
        else:
            starts, labels = [0, 16, 32, 48, 64, 70], [0, 1, 2, 3, -1]
        rows = [0] * len(RANKED_RANKS)
        for g, lab in enumerate(labels):
            if lab >= 0:
                rows[lab] += starts[g + 1] - starts[g]
        flops = 0
        for pi, p in enumerate(layer):
            A, B, Ap, Bp = [], [], [], []
            for j, r in enumerate(RANKED_RANKS):
                aj = synth.device_normal_bf16((r, p["K"]), synth.SIGMA_WAB,
                                              synth.extra_adapter_seed(cfg, 0, pi, synth.T_A, j + 1), dev)
                bj = synth.device_normal_bf16((p["N"], r), synth.SIGMA_WAB,
                                              synth.extra_adapter_seed(cfg, 0, pi, synth.T_B, j + 1), dev)
                ap = torch.zeros((synth.RANK, p["K"]), dtype=torch.bfloat16, device=dev)
                ap[:r] = aj
                bp = torch.zeros((p["N"], synth.RANK), dtype=torch.bfloat16, device=dev)
                bp[:, :r] = bj
                A.append(aj), B.append(bj), Ap.append(ap), Bp.append(bp)
                flops += 2 * rows[j] * r * (p["K"] + p["N"])
            p["A"], p["B"], p["Ap"], p["Bp"] = A, B, Ap, Bp
            flops += 2 * M * p["N"] * p["K"]
        scales = [1.0] * len(RANKED_RANKS)
        ws = torch.zeros(max(bd.workspace_bytes(M, p["N"], p["K"], synth.RANK, len(RANKED_RANKS)) for p in layer),
                         dtype=torch.uint8, device=dev)
        outs = {p["N"]: torch.empty((M, p["N"]), dtype=torch.bfloat16, device=dev) for p in layer}
        stream = torch.cuda.current_stream(dev).cuda_stream

        def step(padded):
            for p in layer:
                if padded:
                    st = bd.lora_proj_raw(p["X"].data_ptr(), starts, labels, p["W"].data_ptr(),
                                          [t.data_ptr() for t in p["Ap"]], [t.data_ptr() for t in p["Bp"]],
                                          synth.RANK, scales, outs[p["N"]].data_ptr(), M, p["N"], p["K"], "bf16",
                                          ws.data_ptr(), ws.numel(), stream)
                else:
                    st = bd.lora_proj_ranked_raw(p["X"].data_ptr(), starts, labels, p["W"].data_ptr(),
                                                 [t.data_ptr() for t in p["A"]], [t.data_ptr() for t in p["B"]],
                                                 RANKED_RANKS, scales, outs[p["N"]].data_ptr(), M, p["N"], p["K"],
                                                 "bf16", ws.data_ptr(), ws.numel(), stream)
                if st != bd.LORA_OK:
                    raise bd.LoraError(st, bd.status_string(st))

        res = {}
        for padded in (False, True):
            for _ in range(a.warmup):
                step(padded)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(a.steps):
                step(padded)
            torch.cuda.synchronize()
            res["padded" if padded else "ranked"] = (time.perf_counter() - t0) * 1e3 / a.steps
        log(f"ranked {path}: {res['ranked']:.3f} ms/step with compact factors, {res['padded']:.3f} zero-padded "
            f"to rank {synth.RANK}")
        out[path] = dict(ms_per_step=round(res["ranked"], 4), padded_ms_per_step=round(res["padded"], 4),
                         speedup=round(res["padded"] / res["ranked"], 3),
                         tflops=round(flops / (res["ranked"] / 1e3) / 1e12, 2), adapter_rows=rows)
        del layer, ws, outs
        torch.cuda.empty_cache()
    out["workload"] = (f"one layer's 7 projections with four adapters of ranks {', '.join(map(str, RANKED_RANKS))} "
                       "(compact factors, lora_proj_ranked) against the same adapters zero-padded to rank 256; "
                       "prefill: 16384 rows in the 212-segment table of prefill_mixed; decode: 70 rows, 4 x 16 "
                       "adapter rows and 6 base rows")
    return out


def run_decode(a, dev, hip, grouped=False, q4=False):
    import torch
    w5 = synth.WORKLOADS["suffix"]
    tag = ("suffix q4" if q4 else "suffix") + (" grouped" if grouped else "")
    log(f"{tag}: drawing 24 layers on the device")
    layers = []
    for l in range(w5["layers"]):
        projs = device_layer(w5["cfg"], l, w5["M"], dev)
        calls = group_layer(projs) if grouped else projs
        if q4:
            for p in calls:
                p["Wq"], p["Wp"] = synth.device_quantize_q4(p["W"])
                del p["W"]
        layers.append(calls)
    runner = StepRunner(layers, w5["seg_starts"], w5["seg_adapter"], w5["scale"], dev)
    dmain, dshrink, dbytes = runner.work()
    clocks = ClockSampler()
    wall5, _ = time_steps(runner, a.decode_steps, a.warmup, hip, events=False, clocks=clocks)
    ms5 = wall5 * 1e3 / a.decode_steps
    gbs = dbytes / (ms5 / 1e3) / 1e9
    log(f"{tag}: {ms5:.3f} ms/step, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.1%} of HBM)")
    n_calls = len(runner.calls)
    del runner, layers
    torch.cuda.empty_cache()
    if grouped:
        workload = ("suffix, grouped: 24 layers x (q/k/v sliced, o, gate/up sliced, down), "
                    "64 adapter rows + 6 base-only decode rows, r=256")
        if q4:
            workload += "; base weights 4-bit (groups of 128, bf16 scale + zero point), adapter bf16"
    else:
        workload = "suffix: 24 layers x 7 projections, 64 adapter rows + 6 base-only decode rows, r=256"
    return dict(workload=workload,
                value=round(gbs, 1), unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4),
                ms_per_step=round(ms5, 4), bytes_per_step=dbytes, steps=a.decode_steps,
                tflops=round((dmain + dshrink) / (ms5 / 1e3) / 1e12, 2),
                calls_per_step=n_calls, call_avg_us=round(ms5 * 1e3 / n_calls, 2), clocks=clocks.summary())


def run_extract(a, dev):
    """Adapter extraction (lora_extract) from a planted rank-256 change of one q-shaped and one
    down-shaped matrix: ms per matrix, with the change's recovery error as a check."""
    import torch
    out = {}
    for name, N, K in (("q", 5120, 5120), ("down", 5120, 17408)):
        g = torch.Generator(device=dev)
        g.manual_seed(7_000_000 + N + K)
        Wb = (torch.randn((N, K), generator=g, device=dev) * 0.14).to(torch.bfloat16)
        B0 = torch.randn((N, synth.RANK), generator=g, device=dev) * 0.1
        A0 = torch.randn((synth.RANK, K), generator=g, device=dev) * 0.1
        Wa = (Wb.float() + B0 @ A0).to(torch.bfloat16)
        del B0, A0
        l = synth.RANK + 16
        omega = torch.randn((K, l), generator=g, device=dev)
        bd.extract(Wa, Wb, synth.RANK, omega)          # warmup
        torch.cuda.synchronize()
        reps = 5
        t0 = time.perf_counter()
        for _ in range(reps):
            B, A, s = bd.extract(Wa, Wb, synth.RANK, omega)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / reps
        D = Wa.float() - Wb.float()
        err = float(torch.linalg.norm(B @ A - D) / torch.linalg.norm(D))
        log(f"extract {name} {N}x{K}: {ms:.1f} ms per matrix, |BA - D| / |D| = {err:.2e}")
        out[name] = dict(N=N, K=K, rank=synth.RANK, l=l, power_iters=2, ms=round(ms, 2), rel_residual=err)
        del Wa, Wb, omega, B, A, s, D
        torch.cuda.empty_cache()
    return dict(workload="extract: rank-256 factors of a planted change (bf16 weights), l=272, 2 power iterations",
                **out)


def measure_peaks(dev):
    """What this GPU sustains, from probes built here (lora_probe.h): dense bf16 MFMA with no memory
    traffic, a streaming read of 4 GiB (16x the 256 MB MALL, so it comes from HBM), and torch's copy
    of 2 GiB (read + written bytes).  Best of three timed runs each."""
    import torch
    st = torch.cuda.current_stream(dev)
    sink = torch.zeros(1024, dtype=torch.float32, device=dev)

    def best(launch, reps=3):
        launch()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            launch()
            e1.record(st)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        return min(times)

    flop = {}

    def mfma():
        status, f = bd.probe_mfma_bf16_raw(2000, sink.data_ptr(), st.cuda_stream)
        if status != bd.LORA_OK:
            raise bd.LoraError(status, "lora_probe_mfma_bf16")
        flop["f"] = f
    t = best(mfma)
    mfma_tflops = flop["f"] / t / 1e12
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    loops = 10

    def read():
        for _ in range(loops):
            status = bd.probe_read_raw(buf.data_ptr(), buf.numel(), sink.data_ptr(), st.cuda_stream)
            if status != bd.LORA_OK:
                raise bd.LoraError(status, "lora_probe_read")
    read_gbs = loops * buf.numel() / best(read) / 1e9
    del buf
    src = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    copy_gbs = 2 * src.numel() / best(lambda: dst.copy_(src)) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    log(f"measured peaks: MFMA bf16 {mfma_tflops:.0f} TFLOP/s, HBM read {read_gbs:.0f} GB/s, "
        f"copy {copy_gbs:.0f} GB/s (read + write)")
    return dict(mfma_bf16_tflops=round(mfma_tflops, 1), hbm_read_gbs=round(read_gbs, 1),
                hbm_copy_gbs=round(copy_gbs, 1),
                how="probes built here: 4 independent v_mfma_f32_32x32x16_bf16 chains per wave, 16 waves per CU, "
                    "no memory traffic; streaming 16-byte reads of 4 GiB; torch copy of 2 GiB")


# ------------------------------------------------------------------ main
def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--no-decode", action="store_true", help="skip the 24-layer decode stack")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=16384)
    ap.add_argument("--stack-steps", type=int, default=3, help="timed passes of the 24-layer 32k stack")
    ap.add_argument("--only", choices=("all", "prefill", "mixed", "stack32k", "prefill_9b", "prefill_mixed",
                                       "decode", "decode_grouped",
                                       "decode_q4", "ranked", "extract", "peaks"),
                    default="all",
                    help="time one workload only (for profiler runs)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="run a plain device copy of MIB mebibytes (reads MIB, writes MIB) five times and exit; "
                         "calibrates the FETCH_SIZE / WRITE_SIZE counters")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: the projection is measured at one GPU's share "
              f"(requested --gpus {a.gpus}); rows shard across GPUs without any exchange.", file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py is single-process; do not launch it with several ranks", file=sys.stderr)
        return 2

    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.copy_probe:
        n = a.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"copy probe: 5 x {a.copy_probe} MiB read + {a.copy_probe} MiB written")
        return 0
    bd.load()
    hip = HipEvents()
    w = synth.WORKLOADS["prefill16k"]
    pre = run_prefill(a, dev, hip) if a.only in ("all", "prefill") else {}
    pre9 = run_prefill(a, dev, hip, "prefill16k_9b") if a.only in ("all", "prefill_9b") else None
    if pre9 is not None:
        pre9 = dict(workload="prefill16k_9b: one layer of the 9B backbone's stand-in shapes (q,o 4096->4096; "
                             "k,v 4096->1024; gate,up 4096->12288; down 12288->4096), 16384 rows all naming "
                             "the adapter, rank 256",
                    value=round(pre9["value"], 2), unit="TFLOP/s", ms_per_step=round(pre9["ms_per_step"], 4),
                    frac=round(pre9["value"] / PEAK_BF16_TFLOPS, 4),
                    main_kernel_tflops=pre9["roofline"]["achieved"],
                    per_projection_ms=pre9["roofline"]["per_projection_ms"])
    mixed = run_prefill_mixed(a, dev, hip) if a.only in ("all", "prefill_mixed") else None
    cfg3 = run_prefill(a, dev, hip, "mixed") if a.only in ("all", "mixed") else None
    if cfg3 is not None:
        cfg3 = dict(workload="mixed: one adapted layer's 7 projections over 6 base-only decode rows (M=1 each) "
                             "around one 2,048-row adapter prefill chunk (2,054 rows), rank 256",
                    value=round(cfg3["value"], 2), unit="TFLOP/s", ms_per_step=round(cfg3["ms_per_step"], 4),
                    frac=round(cfg3["value"] / PEAK_BF16_TFLOPS, 4), steps=cfg3["steps"],
                    main_kernel_tflops=cfg3["roofline"]["achieved"],
                    main_kernel_frac=cfg3["roofline"]["frac"],
                    per_projection_ms=cfg3["roofline"]["per_projection_ms"],
                    per_projection_min_ms=cfg3["roofline"]["per_projection_min_ms"],
                    clocks=cfg3["roofline"]["clocks"])
    st32 = (run_prefill(a, dev, hip, "stack32k", steps=a.stack_steps, warmup=1)
            if a.only in ("all", "stack32k") else None)
    if st32 is not None:
        st32 = dict(workload="stack32k: 32,768 rows all naming the adapter through 24 adapted layers x 7 "
                             "projections (independent weights per layer), rank 256",
                    ms_per_pass=round(st32["ms_per_step"], 2), target_ms=416.7,
                    value=round(st32["value"], 2), unit="TFLOP/s", frac=round(st32["value"] / PEAK_BF16_TFLOPS, 4),
                    steps=st32["steps"], calls_per_pass=st32["calls"],
                    main_kernel_tflops=st32["roofline"]["achieved"], main_kernel_frac=st32["roofline"]["frac"],
                    per_projection_ms=st32["roofline"]["per_projection_ms"],
                    per_projection_min_ms=st32["roofline"]["per_projection_min_ms"],
                    clocks=st32["roofline"]["clocks"])
    decode = run_decode(a, dev, hip) if a.only in ("all", "decode") and not a.no_decode else None
    grouped = (run_decode(a, dev, hip, grouped=True)
               if a.only in ("all", "decode", "decode_grouped") and not a.no_decode else None)
    q4 = (run_decode(a, dev, hip, grouped=True, q4=True)
          if a.only in ("all", "decode", "decode_q4") and not a.no_decode else None)
    ranked = run_ranked(a, dev) if a.only in ("all", "ranked") else None
    extract = run_extract(a, dev) if a.only in ("all", "extract") else None
    peaks = measure_peaks(dev) if a.only in ("all", "peaks") else None
    hip.close()
    if peaks is not None:
        if pre.get("roofline"):
            pre["roofline"]["measured_peak"] = peaks["mfma_bf16_tflops"]
            pre["roofline"]["frac_of_measured_peak"] = round(pre["roofline"]["achieved"] / peaks["mfma_bf16_tflops"], 4)
        for d in (decode, grouped, q4):
            if d is not None:
                d["frac_of_measured_read"] = round(d["value"] / peaks["hbm_read_gbs"], 4)

    cpu = None
    if not a.no_cpu_baseline:
        log("cpu baseline: fp64 oracle on sampled rows")
        cpu = cpu_baseline(a.cpu_rows)

    value, ms_per_step = pre.get("value"), pre.get("ms_per_step")
    out = dict(metric=METRIC, value=None if value is None else round(value, 2), unit="TFLOP/s", n_gpus=1,
               steps=a.steps, warmup=a.warmup, ms_per_step=None if ms_per_step is None else round(ms_per_step, 4),
               higher_is_better=True, scaling="weak", vs_baseline=None,
               dtype="bf16", data="synthetic",
               config=dict(workload="prefill16k: one adapted layer, 16384 rows all naming the adapter, "
                                    "7 projections (q,k,v,o 5120->5120; gate,up 5120->17408; down 17408->5120), "
                                    "rank 256, s=1",
                           M=w["M"], rank=synth.RANK, flop_per_step=pre.get("flops"), bytes_per_step=pre.get("bytes"),
                           parallelism="single GPU"),
               roofline=pre.get("roofline"), cpu_baseline=cpu, decode=decode, decode_grouped=grouped,
               mixed=cfg3, stack32k=st32,
               prefill_9b=pre9, prefill_mixed=mixed, ranked=ranked, decode_q4_grouped=q4, extract=extract,
               measured_peaks=peaks)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
