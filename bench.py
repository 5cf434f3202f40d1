#!/usr/bin/env python3
"""Throughput of the tiled dense GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload KEY]

(--workload takes a GEMM, grouped GEMM or RMSNorm workload key; the default is
the headline GEMM.)

A step is one call of the C entry point gemm_mkl on the headline workload
(bf16 GEMM M=512 N=5632 K=2048 L=1, ReLU epilogue), i.e. one pass of the whole
path (tiling, LDS-staged prefetch ring, MFMA mainloop, fused epilogue; plus the
split-K reduction when the plan splits K).  Inputs are seeded synthetic
operands resident in HBM before the timed region starts.

The K timed steps are captured into one HIP graph on a stream of their own
and replayed once (--no-graph launches them one by one from the host): the
per-launch host and dispatch cost then stays out of the kernel times, as in a
serving loop that replays captured work.

Prints ONE JSON line with the metric, the roofline of the dominant kernel
(measured with HIP events on the stream the kernels run on) and the CPU
oracle timed on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}   # dense MFMA, 256 CU x 2.4 GHz
HBM_GBS = 8000.0
# device code: a change here invalidates the stored counter readings
KERNEL_SOURCES = ["tiled_dense_gemm_mkl_amd/csrc/gemm_kernels.hpp",
                  "tiled_dense_gemm_mkl_amd/csrc/configs.hpp",
                  "tiled_dense_gemm_mkl_amd/csrc/inst_bf16.hip",
                  "tiled_dense_gemm_mkl_amd/csrc/inst_f16.hip",
                  "tiled_dense_gemm_mkl_amd/csrc/inst_f32.hip"]


RMS_KERNEL_SOURCES = ["tiled_dense_gemm_mkl_amd/csrc/rms_norm.hip"]


def source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_key: str, kernel: str, sources=None):
    """HBM bytes per launch from the committed rocprofv3 counter readings
    (FETCH_SIZE and WRITE_SIZE, scaled by the copy-kernel calibration), if they
    were taken on the current device code and the same kernel (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
        e = d.get("workloads", {}).get(workload_key)
        if not e or e.get("source_hash") != source_hash(sources) or e.get("kernel") != kernel:
            return None
        return int(e["bytes_per_launch"])
    except (OSError, ValueError, KeyError, TypeError):
        return None


def time_steps(step, steps: int, warmup: int, stream, graph: bool = False):
    """Run `warmup` untimed steps, then time exactly `steps` steps on `stream`
    (a synchronize on both sides of the region).  Returns (wall-clock ms per
    step, ms per step from HIP events recorded on `stream`).  With graph=True
    the `steps` calls are first captured into one HIP graph and the timed
    region replays it, so the host issues one launch for all of them."""
    import torch

    torch.cuda.synchronize()   # inputs made on other streams are in place
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(steps):
                step()
        g.replay()   # one untimed replay
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    if g is not None:
        g.replay()
    else:
        for _ in range(steps):
            step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, start.elapsed_time(end) / steps


def cpu_baseline(w, A, B, budget_s: float = 10.0):
    """The oracle as it stands, on this host's cores, on a bounded sample of
    the workload: the first m rows of A in every batch (all of them when a
    whole call takes under about 2 s), repeated until about budget_s seconds
    of CPU work (at least 3 calls); the median call time gives the rate."""
    import numpy as np

    import oracle

    oracle.load()
    # one probe call on a few rows sizes the sample
    m = min(w.M, 8)
    t0 = time.perf_counter()
    oracle.gemm64(np.ascontiguousarray(A[:, :m]), B, w.dtype, w.epilogue)
    per_row = (time.perf_counter() - t0) / m
    m = int(max(1, min(w.M, 2.0 / max(per_row, 1e-9))))
    As = np.ascontiguousarray(A[:, :m])
    flops = 2 * m * w.N * w.K * w.L
    times = []
    while len(times) < 3 or (sum(times) < budget_s and len(times) < 200):
        t0 = time.perf_counter()
        y = oracle.gemm64(As, B, w.dtype, w.epilogue)
        times.append(time.perf_counter() - t0)
        del y
    threads = oracle.threads()
    t = sorted(times)[len(times) // 2]
    what = "the full workload" if m == w.M else f"the first {m} of {w.M} rows of A in every batch"
    return {
        "value": round(flops / t / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(times)} calls on {what} ({m}x{w.N}x{w.K}, L={w.L}), "
                  f"binary64 dot products, median {t:.3f} s per call",
    }


def device_info(dev) -> dict:
    """Name, compute units and clock of the GPU as the runtime reports them."""
    import torch

    pr = torch.cuda.get_device_properties(dev)
    info = {"name": pr.name, "compute_units": pr.multi_processor_count,
            "arch": getattr(pr, "gcnArchName", None)}
    clk = getattr(pr, "clock_rate", None)   # kHz, where the runtime reports it
    if clk:
        info["clock_mhz"] = round(clk / 1e3)
    return info


def cold_cache_rate(w, a, b, c, step_ptrs, steps: int) -> dict:
    """Throughput when every call reads A and B from HBM: calls rotate over
    enough copies of A and B that their total exceeds 512 MiB, twice the
    256 MiB memory-side cache, so no call finds its operands cached."""
    import math

    import torch

    nbytes = a.numel() * a.element_size() + b.numel() * b.element_size()
    copies = max(2, math.ceil((512 << 20) / nbytes) + 1)
    bufs = [(a.clone(), b.clone()) for _ in range(copies)]
    torch.cuda.synchronize()
    ptrs = [(x.data_ptr(), y.data_ptr()) for x, y in bufs]
    for i in range(copies):
        step_ptrs(*ptrs[i])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step_ptrs(*ptrs[i % copies])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del bufs
    return {"value": round(w.flops / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "ms_per_step": round(ms, 6),
            "copies": copies, "bytes_rotated": copies * nbytes}


def copy_calibration(mib: int, steps: int) -> int:
    """A plain device copy of known size (torch.neg, out= a second buffer),
    launched `steps` times: rocprofv3's FETCH_SIZE / WRITE_SIZE for it give the
    factor that turns those counters into bytes."""
    import torch

    dev = torch.device("cuda", 0)
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(steps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": True, "bytes_read": n * 4, "bytes_written": n * 4,
                      "launches": steps}), flush=True)
    return 0


def bench_grouped(args, key: str) -> int:
    """The grouped GEMM (gemm_mkl_grouped) on a grouped workload: same timing,
    roofline and CPU-baseline conventions as the dense path."""
    import numpy as np
    import torch

    import tiled_dense_gemm_mkl_amd as gm
    from tiled_dense_gemm_mkl_amd import workloads

    w = workloads.GROUPED_WORKLOADS[key]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    A, B, offs = workloads.make_grouped_inputs(w)
    a = workloads.storage_to_torch(A, w.dtype).to(dev)
    b = workloads.storage_to_torch(B, w.dtype).to(dev)
    o = torch.from_numpy(offs).to(dev)
    c = torch.empty((w.total_m, w.N), dtype=a.dtype, device=dev)
    dcode, ecode = gm.DTYPE_CODES[w.dtype], gm.EPILOGUE_CODES[w.epilogue]
    stream = torch.cuda.Stream(dev)   # a stream of its own (graph capture needs one)
    sptr = stream.cuda_stream
    ptrs = (a.data_ptr(), b.data_ptr(), c.data_ptr(), o.data_ptr())
    kernel = gm.config_names()[gm.grouped_config(w.G, w.total_m, w.N, w.K, dcode, ecode)] + " grouped"

    def step():
        st = gm.gemm_mkl_grouped(*ptrs, w.G, w.total_m, w.N, w.K, dcode, ecode, sptr, None)
        if st != 0:
            raise gm.GemmMklError(st, gm.status_string(st))

    with torch.cuda.stream(stream):
        ms_per_step, ev_ms = time_steps(step, args.steps, args.warmup, stream, args.graph)
    peak = PEAK_TFLOPS[w.dtype]
    value = w.flops / (ms_per_step * 1e-3) / 1e12
    achieved = w.flops / (ev_ms * 1e-3) / 1e12
    result = {
        "metric": f"GEMM TFLOP/s + % of MFMA peak, {w.name}, 1 MI355X",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded; rows routed to groups by a seeded Dirichlet-multinomial)",
        "config": {"workload": w.name, "G": w.G, "total_m": w.total_m, "N": w.N, "K": w.K,
                   "epilogue": w.epilogue, "group_rows": np.diff(np.concatenate([[0], offs])).tolist(),
                   "kernel": kernel},
        "pct_of_mfma_peak": round(100.0 * value / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": measured_traffic(key, kernel),
                     "algorithmic_bytes": w.algorithmic_bytes, "launch_us": round(ev_ms * 1e3, 3)},
    }
    if not args.no_cpu_baseline:
        import oracle

        oracle.load()
        times = []
        while len(times) < 3:
            t1 = time.perf_counter()
            oracle.gemm_grouped64(A, B, offs, w.dtype, w.epilogue)
            times.append(time.perf_counter() - t1)
        t = sorted(times)[1]
        result["cpu_baseline"] = {"value": round(w.flops / t / 1e12, 6), "unit": "TFLOP/s",
                                  "cores": int(oracle.threads()), "kind": "oracle",
                                  "sample": f"3 whole calls on the full grouped workload, median {t:.2f} s"}
    print(json.dumps(result), flush=True)
    return 0


def bench_rms_norm(args, key: str) -> int:
    """RMSNorm (gemm_mkl_rms_norm) on an RMSNorm workload.  A step is one call
    over all rows; the kernel streams x once and writes y once, so it is
    HBM-bound and its roofline is HBM bandwidth."""
    import torch

    import tiled_dense_gemm_mkl_amd as gm
    from tiled_dense_gemm_mkl_amd import workloads

    w = workloads.RMSNORM_WORKLOADS[key]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    X, W = workloads.make_rms_inputs(w)
    x = workloads.storage_to_torch(X, w.dtype).to(dev)
    wt = workloads.storage_to_torch(W, w.dtype).to(dev)
    y = torch.empty_like(x)
    dcode = gm.DTYPE_CODES[w.dtype]
    stream = torch.cuda.Stream(dev)   # a stream of its own (graph capture needs one)
    sptr = stream.cuda_stream
    xp, wp, yp = x.data_ptr(), wt.data_ptr(), y.data_ptr()
    variant = gm.rms_norm_variant(w.rows, w.hidden, dcode, True)
    kernel = "rms_norm " + gm.rms_norm_variant_names()[variant]

    def step():
        st = gm.gemm_mkl_rms_norm(xp, wp, yp, w.rows, w.hidden, w.eps, dcode, sptr)
        if st != 0:
            raise gm.GemmMklError(st, gm.status_string(st))

    with torch.cuda.stream(stream):
        ms_per_step, ev_ms = time_steps(step, args.steps, args.warmup, stream, args.graph)
    nbytes = w.algorithmic_bytes
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (ev_ms * 1e-3) / 1e9
    result = {
        "metric": f"RMSNorm GB/s (x read + y written + weight), {w.name}, 1 MI355X",
        "value": round(value, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded; x ~ N(0,1))",
        "config": {"workload": w.name, "rows": w.rows, "hidden": w.hidden, "eps": w.eps, "kernel": kernel},
        "us_per_call": round(ms_per_step * 1e3, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 3), "peak": HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_GBS, 4),
                     "traffic": measured_traffic(key, kernel, RMS_KERNEL_SOURCES),
                     "algorithmic_bytes": nbytes, "launch_us": round(ev_ms * 1e3, 3)},
    }
    if not args.no_cpu_baseline:
        import oracle

        oracle.load()
        # a bounded prefix of the rows (the same rows the GPU normalises first),
        # repeated until about 10 s of CPU work
        rows = min(w.rows, 8192)
        Xs, _ = workloads.make_rms_inputs(w, rows=rows)
        times, t_total = [], 0.0
        while t_total < 10.0 or len(times) < 3:
            t1 = time.perf_counter()
            oracle.rms_norm64(Xs, W, w.eps, w.dtype)
            dt = time.perf_counter() - t1
            times.append(dt)
            t_total += dt
        t = sorted(times)[len(times) // 2]
        es = 4 if w.dtype == "f32" else 2
        sample_bytes = es * (2 * rows * w.hidden + w.hidden)
        result["cpu_baseline"] = {"value": round(sample_bytes / t / 1e9, 6), "unit": "GB/s",
                                  "cores": int(oracle.threads()), "kind": "oracle",
                                  "sample": f"{len(times)} calls on the first {rows} rows of the workload, "
                                            f"binary64, median {t * 1e3:.3f} ms per call"}
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="launch every timed step from the host instead of replaying them from one HIP graph")
    ap.add_argument("--cold", action="store_true",
                    help="also time calls that rotate over copies of A and B larger than the caches")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run only a device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the library runs each GEMM on a single GPU and has no multi-GPU path", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        return copy_calibration(args.calibrate_copy, max(1, args.steps))

    import torch

    import tiled_dense_gemm_mkl_amd as gm
    from tiled_dense_gemm_mkl_amd import workloads

    key = args.workload or workloads.HEADLINE
    if key in workloads.GROUPED_WORKLOADS:
        return bench_grouped(args, key)
    if key in workloads.RMSNORM_WORKLOADS:
        return bench_rms_norm(args, key)
    w = workloads.WORKLOADS[key]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    A, B = workloads.make_inputs(w)
    a = workloads.storage_to_torch(A, w.dtype).to(dev)
    b = workloads.storage_to_torch(B, w.dtype).to(dev)
    c = torch.empty((w.L, w.M, w.N), dtype=a.dtype, device=dev)
    dcode = gm.DTYPE_CODES[w.dtype]
    ecode = gm.EPILOGUE_CODES[w.epilogue]
    plan = gm.get_plan(w.M, w.N, w.K, w.L, dcode, ecode)
    stream = torch.cuda.Stream(dev)   # a stream of its own (graph capture needs one)
    sptr = stream.cuda_stream
    ap_, bp_, cp_ = a.data_ptr(), b.data_ptr(), c.data_ptr()

    def step_ptrs(ap, bp):
        st = gm.gemm_mkl(ap, bp, cp_, w.M, w.N, w.K, w.L, dcode, ecode, sptr)
        if st != 0:
            raise gm.GemmMklError(st, gm.status_string(st))

    def step():
        step_ptrs(ap_, bp_)

    # HIP events on the stream the kernels run on bracket the K launches: the
    # launches queue back to back, so their span over K is the average launch
    # duration the roofline uses (rocprofv3's kernel trace of the same command
    # shows no idle gap between consecutive launches).  The wall clock over
    # the same region gives the throughput.
    with torch.cuda.stream(stream):
        ms_per_step, ev_ms_per_launch = time_steps(step, args.steps, args.warmup, stream, args.graph)

    value = w.flops / (ms_per_step * 1e-3) / 1e12
    achieved = w.flops / (ev_ms_per_launch * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    kernel_config = gm.config_names()[plan["config_id"]] if plan["config_id"] >= 0 else "general"
    kernel = (f"{kernel_config} P{plan['prefetch_stages']} S{plan['split_k']}" + (" stream-K" if plan["streamk"] else "")
              + (" fix-up" if plan.get("fixup") else ""))
    traffic = measured_traffic(key, kernel)

    result = {
        "metric": ("GEMM TFLOP/s + % of MFMA peak, bf16 M=512 N=5632 K=2048 ReLU, 1 MI355X" if key == workloads.HEADLINE
                   else f"GEMM TFLOP/s + % of MFMA peak, {w.name}, 1 MI355X"),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; A ~ N(0,1), B ~ N(0,0.02^2) for the headline)",
        "config": {
            "workload": w.name,
            "M": w.M, "N": w.N, "K": w.K, "L": w.L,
            "epilogue": w.epilogue,
            "plan": {k: plan[k] for k in ("config_id", "prefetch_stages", "split_k", "grid",
                                           "block_m", "block_n", "block_k", "threads")},
            "kernel": kernel,
        },
        "pct_of_mfma_peak": round(100.0 * value / peak, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "algorithmic_bytes": w.algorithmic_bytes,
            "launch_us": round(ev_ms_per_launch * 1e3, 3),
        },
    }
    result["device"] = device_info(dev)
    if args.cold:
        result["cold_cache"] = cold_cache_rate(w, a, b, c, step_ptrs, args.steps)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, A, B)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
