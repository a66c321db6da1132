"""Throughput of the mixed-precision GEMM on one MI355X.

Default workload: BF16 8192 x 8192 x 8192, row-major A and B, C FP32 N(0,1), alpha = 1,
beta = 0.5, FP32 accumulation and output -- the largest of the five measured configurations.
One step is one D = alpha * A * B + beta * C GEMM on inputs already resident in device memory.

Prints one JSON line:
  * ``value`` / ``ms_per_step``: wall clock over exactly ``--steps`` back-to-back steps, after
    ``--warmup`` steps plus however many more it takes to reach ``--settle`` seconds of warm-up
    (the chip's clock needs about half a second to settle at its power limit);
  * ``roofline``: the GEMM kernel's algorithmic flops per launch over its steady-state launch
    duration -- the median over batches of back-to-back launches timed with HIP events on the
    launch stream, covering at least ``--settle`` seconds after another ``--settle`` seconds of
    warm-up, independent of ``--steps``;
  * ``counters``: MFMA-busy share and HBM GB/s from the committed rocprofv3 counter summary of
    this workload (``profiles/mpgemm_<workload>_counters.txt``) when it was taken on the
    current kernel sources, else null;
  * ``clock``: the shader clock and socket power sampled (amdsmi) during the event timing;
  * ``cpu_baseline``: the CPU oracle on a bounded sample of the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]
  python bench.py --all                           # also one record per configuration (stderr)
  python bench.py --workload f32_4096_nt_bf16x3   # FP32 GEMM as three BF16 products
  python bench.py --workload e4m3_4096_nt         # FP8 E4M3 inputs
  python bench.py --workload f16_sp24_4096_nt     # 2:4 structured-sparse FP16 A
  python bench.py --copy-calibration   # a plain copy of known size, for counter scaling
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "i8": 5000.0, "e4m3": 5000.0,
               "e5m2": 5000.0}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
NUM_SIMDS = 256 * 4              # 256 CUs x 4 SIMDs
NUM_XCDS = 8
MAX_CLOCK_GHZ = 2.4              # MI355X peak engine clock
DEFAULT_WORKLOAD = "bf16_8192_nn"


def kernel_source_digest(sparse: bool = False) -> str:
    """First 16 hex digits of a SHA-256 over the sources a workload's kernel is built from: all
    of csrc/ for the 2:4 sparse kernel, all but the sparse kernel's own files (sp24*) for the
    dense kernels, so that a change to one family leaves the other's recorded counters valid."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "mixed_precision_dense_amd", "csrc", "*"))):
        if not sparse and os.path.basename(p).startswith("sp24"):
            continue
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"mpgemm_{workload}_counters.txt")


def recorded_counters(w):
    """Figures of the committed rocprofv3 counter summary of workload ``w``: a dict, or None
    when the summary is missing or was taken on other kernel sources.

    mfma_busy_pct = SQ_VALU_MFMA_BUSY_CYCLES (summed over the chip's 1024 SIMDs) over
    1024 x (GRBM_GUI_ACTIVE summed over the 8 XCDs / 8), i.e. the share of the dispatch's
    active cycles in which an average SIMD's matrix core was busy;
    hbm_GBs = (FETCH_SIZE x fetch scale + WRITE_SIZE x write scale) x 1024 bytes over the
    rocprofv3 average kernel duration; the scales come from a plain copy of known size.

    GRBM_GUI_ACTIVE counts over a window somewhat longer than the kernel itself, which matters
    only for short kernels.  When the clock it implies over the rocprofv3 duration exceeds the
    chip's 2.4 GHz, that window is evidently longer than the kernel: the clock is then reported
    as null and the MFMA-busy share is marked as a lower bound."""
    workload = w.name
    path = counters_path(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                kv[key.strip()] = val.strip().split()[0] if val.strip() else ""
    if kv.get("workload") != workload or kv.get("kernel_source_sha256") != kernel_source_digest(w.sparse24):
        return None
    try:
        busy = float(kv["sq_SQ_VALU_MFMA_BUSY_CYCLES"])
        active = float(kv["sq_GRBM_GUI_ACTIVE"]) / NUM_XCDS
        dur_ns = float(kv["rocprof_avg_ns"])
        traffic = float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None
    clock = active / dur_ns
    rec = {"file": os.path.relpath(path, ROOT),
           "mfma_busy_pct": round(100.0 * busy / (NUM_SIMDS * active), 2),
           "hbm_GBs": round(traffic / (dur_ns * 1e-9) / 1e9, 1),
           "hbm_bytes_per_launch": traffic,
           "rocprof_avg_us": round(dur_ns / 1e3, 2),
           "clock_GHz_from_counters": round(clock, 3) if clock <= MAX_CLOCK_GHZ else None}
    if clock > MAX_CLOCK_GHZ:
        rec["counter_window_note"] = (
            f"GRBM_GUI_ACTIVE over the kernel's duration implies {clock:.2f} GHz, above the "
            f"chip's {MAX_CLOCK_GHZ} GHz: the counted window is longer than this short kernel, "
            "so mfma_busy_pct is a lower bound")
    return rec


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5) -> None:
    """A device-to-device copy of known size (for scaling FETCH_SIZE / WRITE_SIZE)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


class ClockSampler:
    """Samples the shader clock (MHz, mean over the XCDs that report one) and the socket power
    (W) through amdsmi in a background thread; reports medians.  Leaves ``error`` set and
    reports nothing when amdsmi is not usable."""

    def __init__(self, period_s: float = 0.01):
        self.period = period_s
        self.clk, self.pwr = [], []
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception as e:  # noqa: BLE001 -- any failure just disables sampling
            self.error = f"amdsmi unavailable: {type(e).__name__}"

    def _sample(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        clks = m.get("current_gfxclks")
        vals = [c for c in clks if isinstance(c, int) and 0 < c < 10000] if isinstance(clks, list) else []
        if not vals:
            c = m.get("current_gfxclk")
            vals = [c] if isinstance(c, int) and 0 < c < 10000 else []
        if vals:
            self.clk.append(sum(vals) / len(vals))
        p = m.get("current_socket_power")
        if not isinstance(p, int):
            p = m.get("average_socket_power")
        if isinstance(p, int) and 0 < p < 5000:
            self.pwr.append(p)

    def _run(self):
        while not self._stop.is_set():
            try:
                self._sample()
            except Exception as e:  # noqa: BLE001
                self.error = f"amdsmi sample failed: {type(e).__name__}"
                return
            time.sleep(self.period)

    def __enter__(self):
        if self.error is None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        return False

    def report(self) -> dict:
        if not self.clk:
            return {"gfx_MHz_median": None, "socket_W_median": None,
                    "note": self.error or "no samples"}
        return {"gfx_MHz_median": round(statistics.median(self.clk), 1),
                "socket_W_median": round(statistics.median(self.pwr), 1) if self.pwr else None,
                "samples": len(self.clk), "source": "amdsmi gpu metrics during the event timing"}


def settle(step, min_steps: int, min_s: float) -> tuple:
    """Untimed steps: at least ``min_steps`` and at least ``min_s`` seconds of GPU work.
    Returns (steps run, seconds)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < min_steps:
        step()
        n += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_s:
        for _ in range(8):
            step()
        n += 8
        torch.cuda.synchronize()
    return n, time.perf_counter() - t0


def wall_time(step, steps: int) -> float:
    """Wall-clock ms per step over exactly ``steps`` back-to-back steps."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def event_time(step, stream, min_s: float, est_ms: float, sampler=None) -> dict:
    """Steady-state ms per launch: batches of back-to-back launches bracketed by HIP events
    recorded on the launch stream, each batch about 25 ms, until at least ``min_s`` seconds
    (and at least 5 batches); the median of the batches' per-launch times."""
    import torch
    per_batch = max(1, int(25.0 / max(est_ms, 1e-3)))
    per_launch = []
    total_ms = 0.0
    ctx = sampler if sampler is not None else _Null()
    with ctx:
        while total_ms < min_s * 1e3 or len(per_launch) < 5:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(per_batch):
                step()
            e1.record(stream)
            e1.synchronize()
            ms = e0.elapsed_time(e1)
            total_ms += ms
            per_launch.append(ms / per_batch)
    return {"median_ms": statistics.median(per_launch), "mean_ms": statistics.fmean(per_launch),
            "min_ms": min(per_launch), "max_ms": max(per_launch), "batches": len(per_launch),
            "launches_per_batch": per_batch, "seconds": round(total_ms / 1e3, 3)}


class _Null:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


def cold_time(step, stream, reps: int) -> float:
    """Median ms of single launches, each after 512 MiB written through the caches."""
    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    for _ in range(reps):
        flush.fill_(1)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        step()
        c1.record(stream)
        c1.synchronize()
        cold.append(c0.elapsed_time(c1))
    del flush
    return statistics.median(cold)


def make_step(w, h, inputs=None):
    """Device buffers of ``w``'s inputs and a closure that queues one GEMM on torch's current
    stream.  Returns (step, stream, dD)."""
    import torch
    import mixed_precision_dense_amd as mp
    from gemm_inputs import generate

    inp = generate(w) if inputs is None else inputs
    dA = mp.device_buffer(inp.A, w.in_type)
    dB = mp.device_buffer(inp.B, w.b_type)
    dC = mp.device_buffer(inp.C, w.out_type) if inp.C is not None else None
    dM = mp.device_buffer(inp.meta, "i8") if w.sparse24 else None
    ob = {"f32": 4, "i32": 4, "f16": 2, "bf16": 2}[w.out_type]
    dD = torch.empty(w.m * w.ldc * ob, dtype=torch.uint8, device="cuda")
    compute = "i32" if w.in_type == "i8" else "f32"
    alpha = int(w.alpha) if compute == "i32" else w.alpha
    beta = int(w.beta) if compute == "i32" else w.beta
    stream = torch.cuda.current_stream()

    def step():
        if w.sparse24:
            mp.mpgemm_run_sp24(h.h, w.transb, w.m, w.n, w.k, alpha, dA, w.in_type, w.lda, dM,
                               w.ld_meta, dB, w.b_type, w.ldb, beta, dC, w.out_type, w.ldc, dD,
                               compute, stream=stream)
        else:
            mp.mpgemm_run(h.h, w.transa, w.transb, w.m, w.n, w.k, alpha, dA, w.in_type, w.lda,
                          dB, w.b_type, w.ldb, beta, dC, w.out_type, w.ldc, dD, compute,
                          stream=stream)

    step.keep = (dA, dB, dC, dM)   # the buffers live as long as the closure
    return step, stream, dD


def time_gemm(w, steps: int, warmup: int, settle_s: float, cold_reps: int = 0):
    """Returns a dict: warm-up, wall ms per step over exactly ``steps`` steps, the steady-state
    event timing, the clock during it, the median cold-cache launch, the tile."""
    import mixed_precision_dense_amd as mp

    h = mp.Handle()
    step, stream, _ = make_step(w, h)
    n_warm, warm_s = settle(step, warmup, settle_s)
    wall_ms = wall_time(step, steps)
    settle(step, 0, settle_s)                # warm-up of the event timing
    sampler = ClockSampler()
    ev = event_time(step, stream, settle_s, wall_ms, sampler)
    cold_ms = cold_time(step, stream, cold_reps) if cold_reps else None
    tile = (256, 256) if w.sparse24 else mp.mpgemm_tile_shape(w.m, w.n, w.in_type)
    h.close()
    return {"warmup_steps": n_warm, "warmup_s": warm_s, "wall_ms": wall_ms, "events": ev,
            "clock": sampler.report(), "cold_ms": cold_ms, "tile": tile}


def time_bf16x3(w, steps: int, warmup: int, settle_s: float):
    """FP32 GEMM from BF16 pieces: returns (wall ms per step, ms per step from HIP events for
    the whole call (two split kernels and the GEMM), ms per launch of the GEMM kernel alone on
    the same pieces, tile)."""
    import torch
    import mixed_precision_dense_amd as mp
    from gemm_inputs import generate

    inp = generate(w)
    dA = mp.device_buffer(inp.A, "f32")
    dB = mp.device_buffer(inp.B, "f32")
    dC = mp.device_buffer(inp.C, "f32") if inp.C is not None else None
    dD = torch.empty(w.m * w.ldc * 4, dtype=torch.uint8, device="cuda")
    need = mp.mpgemm_bf16x3_workspace_size(w.transa, w.transb, w.m, w.n, w.k)
    raw = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    ws = (raw.data_ptr() + 255) // 256 * 256
    stream = torch.cuda.current_stream()
    h = mp.Handle()

    def step():
        mp.mpgemm_run_bf16x3(h.h, w.transa, w.transb, w.m, w.n, w.k, w.alpha, dA, w.lda, dB,
                             w.ldb, w.beta, dC, w.ldc, dD, ws, need, stream=stream)

    settle(step, warmup, settle_s)
    wall_ms = wall_time(step, steps)
    settle(step, 0, settle_s)
    call_ms = event_time(step, stream, settle_s, wall_ms)["median_ms"]
    # the GEMM kernel alone, on the pieces the last call left in the workspace
    kp = (w.k + 7) // 8 * 8
    k3 = 3 * kp
    lda3 = (w.m + 7) // 8 * 8 if w.transa else k3
    ldb3 = k3 if w.transb else (w.n + 7) // 8 * 8
    off_b = ((k3 if w.transa else w.m) * lda3 * 2 + 255) // 256 * 256

    def gemm():
        mp.mpgemm_run(h.h, w.transa, w.transb, w.m, w.n, k3, w.alpha, ws, "bf16", lda3,
                      ws + off_b, "bf16", ldb3, w.beta, dC, "f32", w.ldc, dD, "f32",
                      stream=stream)

    gemm_ms = event_time(gemm, stream, settle_s, call_ms)["median_ms"]
    tile = mp.mpgemm_tile_shape(w.m, w.n, "bf16")
    h.close()
    torch.cuda.synchronize()
    return wall_ms, call_ms, gemm_ms, tile


def bf16x3_line(w, args) -> dict:
    wall_ms, call_ms, gemm_ms, tile = time_bf16x3(w, args.steps, args.warmup, args.settle)
    k3 = 3 * ((w.k + 7) // 8 * 8)
    peak = PEAK_TFLOPS["bf16"]
    gemm_flops = 2.0 * w.m * w.n * k3            # the GEMM kernel's algorithmic work
    split_bytes = (4 + 6) * (w.m * w.k + w.k * w.n)   # read FP32, write three BF16 pieces
    split_ms = call_ms - gemm_ms
    line = {
        "metric": "FP32-equivalent TFLOP/s (2mnk per FP32 GEMM) at 1 GPU",
        "value": round(w.flops / (wall_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "m": w.m, "n": w.n, "k": w.k,
                   "transa": "T" if w.transa else "N", "transb": "T" if w.transb else "N",
                   "in": "f32", "products": "3 x bf16 (hi*hi + lo*hi + hi*lo)", "k3": k3,
                   "accumulate": "f32", "out": "f32", "tile": f"{tile[0]}x{tile[1]}",
                   "call_ms_events": round(call_ms, 5), "gemm_ms_events": round(gemm_ms, 5),
                   "split_ms_events": round(split_ms, 5),
                   "split_hbm_GBs": round(split_bytes / (split_ms * 1e-3) / 1e9, 1),
                   "fp32_vector_peak_TFLOPs": 157.3},
        "roofline": {"bound": "mfma", "achieved": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 2),
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / peak, 4),
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_f32(w)
    return line


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_f32(w, target_s: float = 15.0):
    """The oracle's double-precision FP32 GEMM on a bounded sample of output elements."""
    import oracle
    from gemm_inputs import generate, sample_points

    inp = generate(w)
    probe = sample_points(w.m, w.n, 2000, seed=99)
    t0 = time.perf_counter()
    oracle.gemm_f32(w.transa, w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.lda, inp.B, w.ldb,
                    w.beta, inp.C, w.ldc, points=probe)
    per_elem = (time.perf_counter() - t0) / probe[0].size
    count = min(max(int(target_s / per_elem) - 132, 1), w.m * w.n // 2)
    pts = sample_points(w.m, w.n, count, seed=99)
    # repeated over the same sample until at least 10 s of CPU work
    reps, t = 0, 0.0
    while (t < 10.0 and reps < 50) or reps == 0:
        t0 = time.perf_counter()
        oracle.gemm_f32(w.transa, w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.lda, inp.B, w.ldb,
                        w.beta, inp.C, w.ldc, points=pts)
        t += time.perf_counter() - t0
        reps += 1
    return {"value": 2.0 * reps * pts[0].size * w.k / t / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu": cpu_model(),
            "sample": (f"{reps} pass(es) over {pts[0].size} output elements of the "
                       f"{w.m}x{w.n}x{w.k} workload, each a {w.k}-term FP32 dot product in "
                       f"double; {t:.1f} s")}


def oracle_call(w, inp, pts):
    """The oracle's reference for ``w`` (full output when pts is None)."""
    import oracle
    if w.sparse24 and w.in_type == "i8":
        return oracle.gemm_sp24_int(w.transb, w.m, w.n, w.k, int(w.alpha), inp.A, w.lda, inp.meta,
                                    w.ld_meta, inp.B, w.ldb, int(w.beta), inp.C, w.ldc, points=pts)
    if w.sparse24:
        return oracle.gemm_sp24(w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.in_type, w.lda,
                                inp.meta, w.ld_meta, inp.B, w.ldb, w.beta, inp.C, w.out_type,
                                w.ldc, points=pts, btype=w.b_type)
    if w.in_type == "i8":
        return oracle.gemm_int(w.transa, w.transb, w.m, w.n, w.k, int(w.alpha), inp.A, w.lda,
                               inp.B, w.ldb, int(w.beta), inp.C, w.ldc, points=pts)
    if w.in_type in oracle.FP8:
        return oracle.gemm_fp8(w.transa, w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.in_type,
                               w.lda, inp.B, w.b_type, w.ldb, w.beta, inp.C, w.out_type, w.ldc,
                               points=pts)
    return oracle.gemm_fp(w.transa, w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.in_type, w.lda,
                          inp.B, w.in_type, w.ldb, w.beta, inp.C, w.out_type, w.ldc, points=pts)


def _row_band(w, inp, rows: int):
    """The workload restricted to the first ``rows`` rows of D (and of op(A), C, metadata)."""
    from dataclasses import replace
    from gemm_inputs import Inputs
    wb = replace(w, m=rows)
    A = inp.A if w.transa else inp.A[:rows]
    C = None if inp.C is None else inp.C[:rows]
    meta = None if inp.meta is None else inp.meta[:rows]
    return wb, Inputs(wb, A, inp.B, C, meta=meta)


def cpu_baseline(w, target_s: float = 12.0):
    """The oracle, as is, on a bounded sample of the workload: whole passes over the full
    output when one pass fits the time budget, else its full-output path on a band of the
    first rows of D, sized to the budget."""
    import oracle
    from gemm_inputs import generate

    inp = generate(w)
    unit = "TFLOP/s" if w.in_type != "i8" else "TOP/s"
    elem = ("int64 dot product" if w.in_type == "i8"
            else "fp64 dot product plus its sum of |a*b| for the error bound")

    def run(rows):
        wb, ib = _row_band(w, inp, rows)
        t0 = time.perf_counter()
        oracle_call(wb, ib, None)
        return time.perf_counter() - t0

    probe_rows = min(w.m, 16)
    per_row = run(probe_rows) / probe_rows            # calibrate the band
    if per_row * w.m <= target_s:
        # whole passes over the m x n output, repeated until at least 10 s of CPU work
        reps, t = 0, 0.0
        while (t < 10.0 and reps < 50) or reps == 0:
            t += run(w.m)
            reps += 1
        npts = reps * w.m * w.n
        what = f"{reps} full pass(es) over the {w.m}x{w.n}x{w.k} workload's output"
    else:
        rows = max(1, min(w.m, int(target_s / per_row)))
        t = run(rows)
        npts = rows * w.n
        what = (f"the first {rows} of {w.m} rows of the {w.m}x{w.n}x{w.k} workload's output "
                f"({npts} elements, the oracle's full-output path)")
    terms = w.k // 2 if w.sparse24 else w.k
    if w.sparse24:
        elem += " over the kept values of a 2:4 sparse row"
    return {"value": 2.0 * npts * terms / t / 1e12, "unit": unit,
            "cores": oracle.num_threads(), "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{what}; each element a {terms}-term {elem}; {t:.1f} s"}


def config_record(w, args) -> dict:
    """One configuration's record: kernel time (steady-state events), throughput and share of
    peak, the counter figures when a summary for the current sources exists, and parity of the
    full output against the oracle with the oracle's own time on the host cores."""
    import numpy as np
    import torch
    import mixed_precision_dense_amd as mp
    import oracle
    from gemm_inputs import generate

    inp = generate(w)
    h = mp.Handle()
    step, stream, dD = make_step(w, h, inp)
    settle(step, args.warmup, args.settle)
    ev = event_time(step, stream, args.settle, 1.0)
    torch.cuda.synchronize()
    ob = {"f32": 4, "i32": 4, "f16": 2, "bf16": 2}[w.out_type]
    storage = {"f16": np.uint16, "bf16": np.uint16, "f32": np.float32, "i32": np.int32}[w.out_type]
    D = dD.cpu().numpy()[: w.m * w.ldc * ob].view(storage).reshape(w.m, w.ldc)[:, : w.n]
    h.close()
    t0 = time.perf_counter()
    ref = oracle_call(w, inp, None)
    oracle_s = time.perf_counter() - t0
    D = np.ascontiguousarray(D)
    if w.in_type == "i8":
        rep = oracle.check_int(D, ref)
        parity = {"mode": "bit-exact", "n": rep.n, "n_bad": rep.n_bad}
    else:
        rep = oracle.check_fp(D, w.out_type, ref, w.k // 2 if w.sparse24 else w.k, w.alpha,
                              fp8=w.in_type in oracle.FP8)
        parity = {"mode": "bound", "n": rep.n, "n_bad": rep.n_bad,
                  "worst_err_over_bound": round(rep.worst_ratio, 4)}
    pk = PEAK_TFLOPS[w.in_type]
    tf = w.flops / (ev["median_ms"] * 1e-3) / 1e12
    rec = {"workload": w.name, "kernel_ms_median": round(ev["median_ms"], 5),
           "TFLOPs": round(tf, 2), "pct_of_peak": round(100 * tf / pk, 2),
           "counters": recorded_counters(w), "parity_full_output": parity,
           "oracle_full_s": round(oracle_s, 4), "oracle_threads": oracle.num_threads(),
           "oracle_GFLOPs": round(w.flops / oracle_s / 1e9, 2)}
    if w.flops <= 2 * 256 ** 3:
        # the smallest configuration is also timed on one host thread
        threads = oracle.num_threads()
        oracle.set_num_threads(1)
        t0 = time.perf_counter()
        oracle_call(w, inp, None)
        t1 = time.perf_counter() - t0
        oracle.set_num_threads(threads)
        rec["oracle_1thread_s"] = round(t1, 4)
        rec["oracle_1thread_GFLOPs"] = round(w.flops / t1 / 1e9, 2)
    return rec


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of warm-up before each timing, and of event timing")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--all", action="store_true",
                    help="also one record per configuration, full-output parity included "
                         "(one JSON line each on stderr)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the GEMM is measured on "
              "a single MI355X; a multi-GPU run would shard D by output blocks and is not "
              "built.", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration()
        return 0

    from gemm_inputs import NEXT_WORKLOADS, WORKLOADS
    w = WORKLOADS[args.workload] if args.workload in WORKLOADS else NEXT_WORKLOADS[args.workload]
    if w.in_type == "f32":
        print(json.dumps(bf16x3_line(w, args)), flush=True)
        return 0
    t = time_gemm(w, args.steps, args.warmup, args.settle,
                  cold_reps=max(5, min(args.steps // 10, 30)))
    flops = w.flops
    wall_ms = t["wall_ms"]
    value = flops / (wall_ms * 1e-3) / 1e12
    kern_ms = t["events"]["median_ms"]
    achieved = flops / (kern_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.in_type]
    unit = "TOP/s" if w.in_type == "i8" else "TFLOP/s"
    ctr = recorded_counters(w)
    tile = t["tile"]
    line = {
        "metric": "TFLOP/s (TOP/s int8) and % of MI355X dense MFMA peak at 1 GPU",
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.in_type,
        "data": "synthetic",
        "config": {"workload": w.name, "m": w.m, "n": w.n, "k": w.k,
                   "transa": "T" if w.transa else "N", "transb": "T" if w.transb else "N",
                   "in": w.in_type, "in_b": w.b_type,
                   "accumulate": "i32" if w.in_type == "i8" else "f32",
                   "out": w.out_type, "alpha": w.alpha, "beta": w.beta,
                   "tile": f"{tile[0]}x{tile[1]}", "pct_of_peak": round(100 * value / peak, 2),
                   "warmup_steps_run": t["warmup_steps"],
                   "warmup_s": round(t["warmup_s"], 3),
                   "cold_cache_kernel_ms": round(t["cold_ms"], 5),
                   "cold_cache_TFLOPs": round(flops / (t["cold_ms"] * 1e-3) / 1e12, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": ctr["hbm_bytes_per_launch"] if ctr else None,
                     "kernel_ms_median": round(kern_ms, 5),
                     "kernel_ms_mean": round(t["events"]["mean_ms"], 5),
                     "event_batches": t["events"]["batches"],
                     "launches_per_batch": t["events"]["launches_per_batch"],
                     "event_seconds": t["events"]["seconds"]},
        "clock": t["clock"],
        "counters": None,
    }
    if ctr:
        line["counters"] = {
            "mfma_busy_pct": ctr["mfma_busy_pct"], "hbm_GBs": ctr["hbm_GBs"],
            "file": ctr["file"], "rocprof_avg_us": ctr["rocprof_avg_us"],
            "frac_from_rocprof_avg": round(flops / (ctr["rocprof_avg_us"] * 1e-6) / 1e12 / peak, 4),
            "clock_GHz_from_counters": ctr["clock_GHz_from_counters"]}
        if "counter_window_note" in ctr:
            line["counters"]["counter_window_note"] = ctr["counter_window_note"]
    if w.sparse24:
        # the work is the kept products (2 m n k/2); the dense GEMM of the same shape would be
        # twice that
        line["metric"] = (f"{unit} of the kept products (2 m n k/2) of a 2:4 sparse A, and % "
                          "of MI355X dense MFMA peak at 1 GPU")
        line["config"]["sparsity"] = "2:4 on A (kept values m x k/2 plus 2-bit positions)"
        line["config"]["dense_equivalent_" + unit.replace("/", "")] = round(2 * value, 2)
        line["config"]["transa"] = "N"
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    if args.all:
        for wx in WORKLOADS.values():
            print(json.dumps(config_record(wx, args)), file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
