"""Throughput of the mixed-precision GEMM on one MI355X.

Default workload: FP16 4096 x 4096 x 4096, A row-major, B stored n x k (transb = T), beta = 0,
FP32 accumulation and output -- one step is one D = alpha * A * B^T GEMM on inputs already
resident in device memory.  Prints one JSON line with TFLOP/s, the roofline of the GEMM
kernel (MFMA bound, measured with HIP events on the launch stream) and the CPU oracle's rate
on a bounded sample of the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]
  python bench.py --workload f32_4096_nt_bf16x3   # FP32 GEMM as three BF16 products
  python bench.py --workload e4m3_4096_nt         # FP8 E4M3 inputs
  python bench.py --workload f16_sp24_4096_nt     # 2:4 structured-sparse FP16 A
  python bench.py --workload i8_sp24_4096_nn      # 2:4 structured-sparse INT8 A
  python bench.py --workload e4m3_sp24_4096_nt    # 2:4 structured-sparse E4M3 A
  python bench.py --copy-calibration   # a plain copy of known size, for counter scaling
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "i8": 5000.0, "e4m3": 5000.0,
               "e5m2": 5000.0}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "mpgemm_f16_4096_nt_counters.txt")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "mixed_precision_dense_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when the
    summary is missing, for another workload, or taken on different kernel sources."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    kv = {}
    with open(COUNTERS_FILE) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                kv[key.strip()] = val.strip()
    if kv.get("workload") != workload or kv.get("kernel_source_sha256") != kernel_source_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


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


def time_gemm(w, steps: int, warmup: int):
    """Returns (wall ms per step, kernel ms per launch from HIP events, tile, median kernel ms
    per launch with cold caches)."""
    import torch
    import mixed_precision_dense_amd as mp
    from gemm_inputs import generate

    inp = generate(w)
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
    h = mp.Handle()

    def step():
        if w.sparse24:
            mp.mpgemm_run_sp24(h.h, w.transb, w.m, w.n, w.k, alpha, dA, w.in_type, w.lda, dM,
                               w.ld_meta, dB, w.b_type, w.ldb, beta, dC, w.out_type, w.ldc, dD,
                               compute, stream=stream)
        else:
            mp.mpgemm_run(h.h, w.transa, w.transb, w.m, w.n, w.k, alpha, dA, w.in_type, w.lda,
                          dB, w.b_type, w.ldb, beta, dC, w.out_type, w.ldc, dD, compute,
                          stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # wall clock over exactly `steps` steps
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    # kernel time: HIP events recorded on the stream the kernel is launched on
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    ev1.synchronize()
    kern_ms = ev0.elapsed_time(ev1) / steps
    # cold caches: before each timed launch, 512 MiB written through L2 and the last-level cache
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    for _ in range(max(5, min(steps // 10, 30))):
        flush.fill_(1)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        step()
        c1.record(stream)
        c1.synchronize()
        cold.append(c0.elapsed_time(c1))
    del flush
    cold_ms = sorted(cold)[len(cold) // 2]
    tile = (256, 256) if w.sparse24 else mp.mpgemm_tile_shape(w.m, w.n, w.in_type)
    h.close()
    return wall_ms, kern_ms, tile, cold_ms


def time_bf16x3(w, steps: int, warmup: int):
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

    def timed(fn, n):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(n):
            fn()
        ev1.record(stream)
        ev1.synchronize()
        return ev0.elapsed_time(ev1) / n

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    call_ms = timed(step, steps)
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

    gemm_ms = timed(gemm, steps)
    tile = mp.mpgemm_tile_shape(w.m, w.n, "bf16")
    h.close()
    return wall_ms, call_ms, gemm_ms, tile


def bf16x3_line(w, args) -> dict:
    wall_ms, call_ms, gemm_ms, tile = time_bf16x3(w, args.steps, args.warmup)
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


def cpu_baseline(w, target_s: float = 15.0):
    """The oracle, as is, on a bounded sample of the workload: whole passes over the full
    output when one pass fits the time budget, else a sample of output elements."""
    import oracle
    from gemm_inputs import generate, sample_points

    inp = generate(w)
    unit = "TFLOP/s" if w.in_type != "i8" else "TOP/s"
    elem = ("int64 dot product" if w.in_type == "i8"
            else "fp64 dot product plus its sum of |a*b| for the error bound")

    def run(pts):
        t0 = time.perf_counter()
        if w.sparse24 and w.in_type == "i8":
            oracle.gemm_sp24_int(w.transb, w.m, w.n, w.k, int(w.alpha), inp.A, w.lda, inp.meta,
                                 w.ld_meta, inp.B, w.ldb, int(w.beta), inp.C, w.ldc, points=pts)
        elif w.sparse24:
            oracle.gemm_sp24(w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.in_type, w.lda, inp.meta,
                             w.ld_meta, inp.B, w.ldb, w.beta, inp.C, w.out_type, w.ldc,
                             points=pts, btype=w.b_type)
        elif w.in_type == "i8":
            oracle.gemm_int(w.transa, w.transb, w.m, w.n, w.k, int(w.alpha), inp.A, w.lda, inp.B,
                            w.ldb, int(w.beta), inp.C, w.ldc, points=pts)
        elif w.in_type in oracle.FP8:
            oracle.gemm_fp8(w.transa, w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.in_type, w.lda,
                            inp.B, w.b_type, w.ldb, w.beta, inp.C, w.out_type, w.ldc, points=pts)
        else:
            oracle.gemm_fp(w.transa, w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.in_type, w.lda,
                           inp.B, w.in_type, w.ldb, w.beta, inp.C, w.out_type, w.ldc, points=pts)
        return time.perf_counter() - t0

    probe = sample_points(w.m, w.n, 20000, seed=99)
    t = run(probe)                                   # calibrate the sample size
    per_elem = t / probe[0].size
    full_s = per_elem * w.m * w.n
    if full_s <= target_s:
        # whole passes over the m x n output, repeated until at least 10 s of CPU work
        reps, t = 0, 0.0
        while (t < 10.0 and reps < 50) or reps == 0:
            t += run(None)
            reps += 1
        npts = reps * w.m * w.n
        what = (f"{reps} full pass(es) over the {w.m}x{w.n}x{w.k} workload's output")
    else:
        pts = sample_points(w.m, w.n, max(int(target_s / per_elem) - 132, 1), seed=99)
        t = run(pts)
        npts = pts[0].size
        what = (f"{npts} output elements (random points plus the corners, last row and last "
                f"column) of the {w.m}x{w.n}x{w.k} workload")
    terms = w.k // 2 if w.sparse24 else w.k
    if w.sparse24:
        elem += " over the kept values of a 2:4 sparse row"
    return {"value": 2.0 * npts * terms / t / 1e12, "unit": unit,
            "cores": oracle.num_threads(), "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{what}; each element a {terms}-term {elem}; {t:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="f16_4096_nt")
    ap.add_argument("--all", action="store_true",
                    help="also time every named workload (one line each on stderr)")
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
    wall_ms, kern_ms, tile, cold_ms = time_gemm(w, args.steps, args.warmup)
    flops = w.flops
    value = flops / (wall_ms * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.in_type]
    unit = "TOP/s" if w.in_type == "i8" else "TFLOP/s"
    traffic = recorded_traffic(w.name)
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
                   "cold_cache_kernel_ms": round(cold_ms, 5),
                   "cold_cache_TFLOPs": round(flops / (cold_ms * 1e-3) / 1e12, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic},
    }
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
        for name, wx in WORKLOADS.items():
            wm, km, tl, _ = time_gemm(wx, max(10, args.steps // 2), args.warmup)
            pk = PEAK_TFLOPS[wx.in_type]
            rec = {"workload": name, "kernel_ms": round(km, 5), "wall_ms": round(wm, 5),
                   "tflops_kernel": round(wx.flops / km / 1e9, 2),
                   "pct_peak_kernel": round(100 * wx.flops / km / 1e9 / pk, 2),
                   "tile": f"{tl[0]}x{tl[1]}"}
            print(json.dumps(rec), file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
