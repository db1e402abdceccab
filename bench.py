#!/usr/bin/env python3
"""Throughput of linrec_scan on one MI355X, printed as one JSON line.

A step is one linrec_scan call over one batch of the chosen workload (default:
B=32, L=4096, D=256 fp32, a ~ U(0,1), b ~ N(0,1), seeded), inputs already in
HBM.  Several copies of the inputs and outputs are rotated so that successive
steps do not find their data in the 256 MB Infinity Cache.  ``value`` is the
algorithmic HBM throughput, 12 bytes per element (read a, read b, write h),
over the wall time of exactly --steps steps bracketed by device
synchronisation.  ``roofline.achieved`` uses the same bytes over the average
kernel duration measured with HIP events on the launch stream.

The CPU baseline leg times the float64 oracle on the same host arrays for a
bounded number of seconds and checks the last GPU output against it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

import numpy as np  # noqa: E402

import linrec_inputs as li  # noqa: E402

PEAK_HBM_GBS = 8000.0
METRIC = "achieved HBM GB/s and % of peak, linrec_scan B=32 L=4096 D=256 fp32"
KERNEL_SOURCES = [
    ROOT / "linear_recurrence_scan_linrec_amd" / "csrc" / "linrec.hip",
    ROOT / "linear_recurrence_scan_linrec_amd" / "csrc" / "scan_kernel.hpp",
    ROOT / "include" / "linrec.h",
]
TRAFFIC_FILE = ROOT / "profiles" / "traffic_scan_tiles_pages_shape.json"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(p.read_bytes())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were taken on
    the current kernel source and this workload; otherwise None."""
    if not TRAFFIC_FILE.exists():
        return None
    rec = json.loads(TRAFFIC_FILE.read_text())
    if rec.get("kernel_source_sha256") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    return int(rec["hbm_bytes_per_launch"])


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=li.HEADLINE, choices=sorted(li.WORKLOADS))
    p.add_argument("--sets", type=int, default=0, help="input/output copies to rotate (0: enough for >= 1 GB)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="time budget of the oracle baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


def cpu_baseline(a_np, b_np, h_last, seconds: float, shape):
    import oracle

    threads = oracle.default_threads()
    n = a_np.size
    passes, ref = 0, None
    t0 = time.perf_counter()
    while True:
        ref = oracle.linrec_oracle_f64(a_np, b_np, threads=threads)
        passes += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= seconds:
            break
    gbs = 12.0 * n * passes / elapsed / 1e9
    ratio = np.abs(h_last.astype(np.float64) - ref) / (1.0 + np.abs(ref))
    B, L, D = shape
    return {
        "value": round(gbs, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{passes} full passes of the B={B} L={L} D={D} workload in {elapsed:.1f} s "
                  f"(float64 sequential loop, 12 B/element basis)",
        "elements_per_s": round(n * passes / elapsed, 1),
        "gpu_check_max_ratio": float(ratio.max()),
    }


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported by this build "
              "(the scan shards over batch rows and channels with no communication; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_recurrence_scan_linrec_amd import linrec as lr

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    w = li.WORKLOADS[args.workload]
    seed = w.seeds[0]
    a_np, b_np = li.workload_inputs(args.workload, seed)
    n = a_np.size
    step_bytes = 12 * n
    sets = args.sets if args.sets > 0 else max(1, math.ceil(1.0e9 / step_bytes))
    a0 = torch.from_numpy(a_np).cuda()
    b0 = torch.from_numpy(b_np).cuda()
    a_sets = [a0] + [a0.clone() for _ in range(sets - 1)]
    b_sets = [b0] + [b0.clone() for _ in range(sets - 1)]
    h_sets = [torch.empty_like(a0) for _ in range(sets)]
    stream = torch.cuda.current_stream()
    plan = lr.linrec_scan_plan(w.B, w.L, w.D)

    for i in range(args.warmup):
        k = i % sets
        lr.linrec_scan(a_sets[k], b_sets[k], h_sets[k], stream=stream)
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        k = (args.warmup + i) % sets
        starts[i].record(stream)
        lr.linrec_scan(a_sets[k], b_sets[k], h_sets[k], stream=stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    last = (args.warmup + args.steps - 1) % sets

    kernel_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (wall / args.steps) / 1e9
    achieved = step_bytes / (kernel_ms.mean() * 1e-3) / 1e9

    out = {
        "metric": METRIC if args.workload == li.HEADLINE else f"achieved HBM GB/s, linrec_scan {w.describe()}",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {w.describe()}",
            "B": w.B, "L": w.L, "D": w.D, "seed": seed,
            "buffer_sets": sets,
            "plan": plan,
        },
        "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        "elements_per_s": round(n / (wall / args.steps), 1),
        "kernel_us": {
            "mean": round(float(kernel_ms.mean()) * 1e3, 2),
            "p10": round(float(np.percentile(kernel_ms, 10)) * 1e3, 2),
            "p50": round(float(np.percentile(kernel_ms, 50)) * 1e3, 2),
            "p90": round(float(np.percentile(kernel_ms, 90)) * 1e3, 2),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(args.workload),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        h_last = h_sets[last].cpu().numpy()
        out["cpu_baseline"] = cpu_baseline(a_np, b_np, h_last, args.cpu_seconds, (w.B, w.L, w.D))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
