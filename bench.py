#!/usr/bin/env python3
"""Throughput of linrec_scan on one MI355X, printed as one JSON line.

A step is one linrec_scan call over one batch of the chosen workload (default:
B=32, L=4096, D=256 fp32, a ~ U(0,1), b ~ N(0,1), seeded), inputs already in
HBM.  Several copies of the inputs and outputs are rotated so that successive
steps do not find their data in the 256 MB Infinity Cache.  ``value`` is the
algorithmic HBM throughput, 12 bytes per element (read a, read b, write h),
over the wall time of exactly --steps steps bracketed by device
synchronisation.  ``roofline.achieved`` uses the same bytes over the average
launch duration: HIP events on the launch stream bracket the timed launches,
which run back to back.

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
# device code only: host-side edits that leave the kernel and its launch plan
# unchanged keep a counter measurement valid
KERNEL_SOURCES = [
    ROOT / "linear_recurrence_scan_linrec_amd" / "csrc" / "scan_kernel.hpp",
]
PROFILES = ROOT / "profiles"


def traffic_file(workload: str) -> Path:
    """The counter record of a workload, named for the kernel its plan launches."""
    kernel = "scan_one" if current_plan(workload)["mode"] == 1 else "scan_tiles"
    return PROFILES / f"traffic_{kernel}_{workload}.json"


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and whitespace removed, so that an edit to
    comments alone keeps a counter measurement valid while any code change voids it."""
    import re

    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        text = re.sub(r"/\*.*?\*/", " ", p.read_text(), flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def current_plan(workload: str) -> dict:
    from linear_recurrence_scan_linrec_amd import linrec as lr

    w = li.WORKLOADS[workload]
    return lr.linrec_scan_plan(w.B, w.L, w.D)


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were taken on
    the current kernel source, launch plan and workload; otherwise None."""
    path = traffic_file(workload)
    if not path.exists():
        return None
    rec = json.loads(path.read_text())
    if (rec.get("kernel_source_sha256") != kernel_source_hash() or rec.get("workload") != workload
            or rec.get("plan") != current_plan(workload)):
        return None
    return int(rec["hbm_bytes_per_launch"])


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=li.HEADLINE, choices=sorted(li.WORKLOADS))
    p.add_argument("--dtype", default="f32", choices=["f32", "bf16", "f16"],
                   help="storage type of a, b and h (arithmetic is fp32); not f32 runs linrec_scan_ex")
    p.add_argument("--reverse", action="store_true", help="the reverse-time recurrence (linrec_scan_ex)")
    p.add_argument("--state", action="store_true", help="pass an initial state and ask for the final state")
    p.add_argument("--sets", type=int, default=0, help="input/output copies to rotate (0: enough for >= 1 GB, at most warmup + steps)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="time budget of the oracle baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibration-copy", type=int, default=0, metavar="N",
                   help="after the timed steps, run N plain device copies of 512 MiB (known bytes) so that "
                        "rocprofv3 FETCH_SIZE/WRITE_SIZE can be scaled against them")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no GPU work: turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, then "
                        "WRITE_SIZE) of a run with --calibration-copy into the HBM bytes per scan launch, "
                        "written to profiles/ for the roofline's traffic field")
    return p.parse_args()


CALIBRATION_BYTES = 512 * 1024 * 1024


def counters_by_kernel(path, counter):
    import csv

    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            name = row["Kernel_Name"]
            key = "scan" if ("scan_tiles" in name or "scan_one" in name) else ("copy" if "copyBuffer" in name else None)
            if key is not None:
                out.setdefault(key, []).append(float(row["Counter_Value"]) * 1024.0)   # KiB -> bytes
    return out


def traffic_record(fetch, write, workload):
    """The traffic record from per-dispatch counter bytes (``counters_by_kernel`` of the FETCH_SIZE
    and the WRITE_SIZE run): each counter is scaled by what it reads for a copy of known size."""
    for name, d in (("FETCH_SIZE", fetch), ("WRITE_SIZE", write)):
        if "scan" not in d or "copy" not in d:
            raise SystemExit(f"{name}: need both scan kernel and copyBuffer dispatches in the csv")
    f_factor = CALIBRATION_BYTES / float(np.mean(fetch["copy"]))
    w_factor = CALIBRATION_BYTES / float(np.mean(write["copy"]))
    read = float(np.mean(fetch["scan"])) * f_factor
    written = float(np.mean(write["scan"])) * w_factor
    w = li.WORKLOADS[workload]
    algorithmic = 12 * w.elements
    rec = {
        "workload": workload,
        "kernel_source_sha256": kernel_source_hash(),
        "plan": current_plan(workload),
        "hbm_bytes_per_launch": int(round(read + written)),
        "read_bytes_per_launch": int(round(read)),
        "written_bytes_per_launch": int(round(written)),
        "algorithmic_bytes_per_launch": algorithmic,
        "fetch_scale": round(f_factor, 4),
        "write_scale": round(w_factor, 4),
        "scan_dispatches": [len(fetch["scan"]), len(write["scan"])],
        "copy_dispatches": [len(fetch["copy"]), len(write["copy"])],
    }
    return rec


def traffic_from(fetch_csv, write_csv, workload):
    """Scale the counters by what they read for a copy of known size; store and print the result."""
    rec = traffic_record(counters_by_kernel(fetch_csv, "FETCH_SIZE"), counters_by_kernel(write_csv, "WRITE_SIZE"),
                         workload)
    traffic_file(workload).write_text(json.dumps(rec, indent=1) + "\n")
    print(json.dumps(rec))


def cpu_baseline(a_np, b_np, h_last, seconds: float, shape, reverse=False, h_init=None):
    import oracle

    threads = oracle.default_threads()
    fn = oracle.linrec_oracle_rev_f64 if reverse else oracle.linrec_oracle_f64
    n = a_np.size
    passes, ref = 0, None
    t0 = time.perf_counter()
    while True:
        ref = fn(a_np, b_np, h_init=h_init, threads=threads)
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
    if args.traffic_from:
        traffic_from(args.traffic_from[0], args.traffic_from[1], args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported.  The scan would shard over "
              "batch rows and channel slabs with no communication, or along L with one exchange of per-channel "
              "carries; neither is built here.", file=sys.stderr)
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
    storage = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[args.dtype]
    elem = 4 if args.dtype == "f32" else 2
    plain = args.dtype == "f32" and not args.reverse and not args.state
    # algorithmic bytes: read a and b, write h, plus the initial and final states
    step_bytes = 3 * elem * n + (8 * w.B * w.D if args.state else 0)
    # enough copies that the rotation spans >= 1 GB (beyond the 256 MB Infinity Cache), but never
    # more than the run uses: a tiny workload would otherwise allocate ~1e5 copies
    sets = args.sets if args.sets > 0 else max(1, min(math.ceil(1.0e9 / step_bytes), args.warmup + args.steps))
    # each set is uploaded from host memory (converted to the storage type on
    # the host: no device-side copy kernels, so the calibration copies are the
    # only copy dispatches in a counter profile)
    a_host = torch.from_numpy(a_np).to(storage)
    b_host = torch.from_numpy(b_np).to(storage)
    a_sets = [a_host.cuda() for _ in range(sets)]
    b_sets = [b_host.cuda() for _ in range(sets)]
    h_sets = [torch.empty_like(a_sets[0]) for _ in range(sets)]
    h0_np = np.random.default_rng(seed + 1000).standard_normal((w.B, w.D)).astype(np.float32) if args.state else None
    h0 = torch.from_numpy(h0_np).cuda() if args.state else None
    hf = torch.empty((w.B, w.D), dtype=torch.float32, device="cuda") if args.state else None
    stream = torch.cuda.current_stream()
    plan = (lr.linrec_scan_plan(w.B, w.L, w.D) if plain else
            lr.plan_for(a_sets[0], b_sets[0], h_sets[0], h_init=h0, h_final=hf, reverse=args.reverse))

    def step(k):
        if plain:
            lr.linrec_scan(a_sets[k], b_sets[k], h_sets[k], stream=stream)
        else:
            lr.linrec_scan(a_sets[k], b_sets[k], h_sets[k], stream=stream, h_init=h0, h_final=hf,
                           reverse=args.reverse)

    for i in range(args.warmup):
        step(i % sets)
    torch.cuda.synchronize()

    # one event pair on the launch stream brackets the timed launches, which run
    # back to back; their average duration is the region's time over --steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step((args.warmup + i) % sets)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    last = (args.warmup + args.steps - 1) % sets

    launch_us = start.elapsed_time(end) * 1e3 / args.steps
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (wall / args.steps) / 1e9
    achieved = step_bytes / (launch_us * 1e-6) / 1e9

    variant = "" if plain else " (linrec_scan_ex: " + ", ".join(
        x for x in (f"{args.dtype} storage" if args.dtype != "f32" else "", "reverse time" if args.reverse else "",
                    "initial and final state" if args.state else "") if x) + ")"
    headline = args.workload == li.HEADLINE and plain
    out = {
        "metric": METRIC if headline else f"achieved HBM GB/s, linrec_scan {w.describe()}{variant}",
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
            "workload": f"{args.workload}: {w.describe()}{variant}",
            "B": w.B, "L": w.L, "D": w.D, "seed": seed,
            "storage": args.dtype, "reverse": args.reverse, "state": args.state,
            "algorithmic_bytes_per_step": step_bytes,
            "buffer_sets": sets,
            "plan": plan,
        },
        "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        "elements_per_s": round(n / (wall / args.steps), 1),
        "launch_us_mean": round(launch_us, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(args.workload) if plain else None,
        },
        "cpu_baseline": None,
    }
    if args.calibration_copy:
        src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.calibration_copy):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        # the oracle on the values the GPU consumed (16-bit inputs widen exactly)
        h_last = h_sets[last].float().cpu().numpy()
        out["cpu_baseline"] = cpu_baseline(a_host.float().numpy(), b_host.float().numpy(), h_last, args.cpu_seconds,
                                           (w.B, w.L, w.D), reverse=args.reverse, h_init=h0_np)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
