#!/usr/bin/env python3
"""Throughput of linrec_scan on one MI355X, printed as one JSON line.

A step is one linrec_scan call over one batch of the chosen workload (default:
B=32, L=4096, D=256 fp32, a ~ U(0,1), b ~ N(0,1), seeded), inputs already in
HBM.  Several copies of the inputs and outputs are rotated so that successive
steps do not find their data in the 256 MB Infinity Cache.  ``value`` is the
algorithmic HBM throughput, 12 bytes per element (read a, read b, write h;
6 with 16-bit storage), over the wall time of exactly --steps steps bracketed
by device synchronisation.  One HIP event pair on the launch stream brackets
the timed launches, which run back to back: ``launch_us.mean`` is that span
over --steps, and ``roofline.achieved`` the algorithmic bytes over it.  (An
event pair around every launch would add 2-7 us to each measured launch on
MI355X, measured against rocprofv3's kernel trace, so none is used there.)

After the timed region (never inside it):
* ``launch_us`` median/p10/p90: the means of --regions further regions of 10
  back-to-back launches, each bracketed the same way.
* ``ceiling``: the read-two-write-one stream z = x + y of libstream_ceiling.so
  over the same buffers (the same bytes and rotation), contiguous and in the
  scan's order over batch rows, each the best of a small sweep of launch
  shapes timed the same way; ``frac_of_ceiling`` is the scan's achieved rate
  over the contiguous stream's.
* ``ceiling.tile_walk`` (fp32 local-carry plans of one sequence per
  workgroup): the same stream in the plan's own tile walk
  (linrec_stream_column_walk: one workgroup per (batch row, channel slab)
  sequence, the plan's waves and rows per lane, two barriers per tile) over the
  same buffers, and the scan's rate over it; ``--walk-shapes`` times other walk
  shapes instead.
* ``--cold N`` (default 10): N single launches, each after a 1 GiB write that
  evicts the caches, and N single warm launches, each with its own event pair
  (so both carry the same per-pair overhead and compare with each other).
* the CPU baseline: the float64 oracle on the same host arrays for a bounded
  number of seconds, multi-threaded and single-threaded, and a check of the
  last GPU output against it at the storage type's bar.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
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
    ROOT / "linear_recurrence_scan_linrec_amd" / "csrc" / "call_epoch.hpp",
]
PROFILES = ROOT / "profiles"


STORAGE_BYTES = {"f32": 4, "bf16": 2, "f16": 2}


def traffic_file(workload: str, dtype: str = "f32") -> Path:
    """The counter record of a workload in a storage type, named for the kernel its plan launches."""
    kernel = {1: "scan_one", 2: "scan_relay"}.get(current_plan(workload, dtype)["mode"], "scan_tiles")
    suffix = "" if dtype == "f32" else f"_{dtype}"
    return PROFILES / f"traffic_{kernel}_{workload}{suffix}.json"


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


def current_plan(workload: str, dtype: str = "f32") -> dict:
    """The plan of a forward scan of the workload over contiguous operands of the storage type
    (host arithmetic only: 16-byte aligned stand-in addresses, nothing is dereferenced)."""
    import ctypes

    from linear_recurrence_scan_linrec_amd import linrec as lr

    w = li.WORKLOADS[workload]
    desc = lr.linrec_scan_desc()
    desc.B, desc.L, desc.D = w.B, w.L, w.D
    desc.dtype = {"f32": lr.LINREC_F32, "bf16": lr.LINREC_BF16, "f16": lr.LINREC_F16}[dtype]
    desc.reverse = 0
    for op in (desc.a, desc.b, desc.h):
        op.ptr, op.stride_b, op.stride_l = 256, w.L * w.D, w.D
    plan = lr.linrec_plan()
    status = lr.library().linrec_scan_ex_plan(ctypes.byref(desc), ctypes.byref(plan))
    if status != lr.LINREC_OK:
        raise RuntimeError(f"linrec_scan_ex_plan: {lr.linrec_last_error_message()}")
    return {name: getattr(plan, name) for name, _ in lr.linrec_plan._fields_}


def measured_traffic(workload: str, dtype: str = "f32"):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were taken on
    the current kernel source, launch plan, workload and storage type; otherwise None."""
    path = traffic_file(workload, dtype)
    if not path.exists():
        return None
    rec = json.loads(path.read_text())
    if (rec.get("kernel_source_sha256") != kernel_source_hash() or rec.get("workload") != workload
            or rec.get("storage", "f32") != dtype or rec.get("plan") != current_plan(workload, dtype)):
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
    p.add_argument("--a-ahead", action="store_true",
                   help="with --reverse: the decays taken one time step ahead (dLoss/db of a forward scan)")
    p.add_argument("--state", action="store_true", help="pass an initial state and ask for the final state")
    p.add_argument("--sets", type=int, default=0, help="input/output copies to rotate (0: enough for >= 1 GB, at most warmup + steps)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="time budget of the multi-threaded oracle baseline")
    p.add_argument("--cpu-single-seconds", type=float, default=5.0, help="time budget of the single-threaded oracle pass")
    p.add_argument("--cold", type=int, default=10, metavar="N",
                   help="after the timed steps, N launches each preceded by a cache-evicting write, and N warm "
                        "ones, each with its own event pair (not part of the timed region; 0: none)")
    p.add_argument("--no-ceiling", action="store_true", help="skip the streaming-ceiling sweep")
    p.add_argument("--ceiling-shape", metavar="R,U,G",
                   help="run the ceiling only in this walk (rows R), unroll U and groups per CU G (for counter runs)")
    p.add_argument("--stream-rows", metavar="R1,R2,...",
                   help="no scan: time the read-2-write-1 stream over this workload's buffers walking R batch-row "
                        "streams at once (R = 1: one contiguous sweep), best launch shape per R; prints one JSON line")
    p.add_argument("--walk-shapes", metavar="P,W,T;...",
                   help="time the stream in these tile walks (lanes per row P, waves W, rows per lane T) instead of "
                        "the plan's own")
    p.add_argument("--regions", type=int, default=10,
                   help="further regions of 10 launches whose means give median/p10/p90 (0: none)")
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
            key = ("scan" if any(k in name for k in ("scan_tiles", "scan_one", "scan_relay"))
                   else ("copy" if "copyBuffer" in name else None))
            if key is not None:
                out.setdefault(key, []).append(float(row["Counter_Value"]) * 1024.0)   # KiB -> bytes
    return out


def traffic_record(fetch, write, workload, dtype="f32"):
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
    algorithmic = 3 * STORAGE_BYTES[dtype] * w.elements
    rec = {
        "workload": workload,
        "storage": dtype,
        "kernel_source_sha256": kernel_source_hash(),
        "plan": current_plan(workload, dtype),
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


def traffic_from(fetch_csv, write_csv, workload, dtype="f32"):
    """Scale the counters by what they read for a copy of known size; store and print the result."""
    rec = traffic_record(counters_by_kernel(fetch_csv, "FETCH_SIZE"), counters_by_kernel(write_csv, "WRITE_SIZE"),
                         workload, dtype)
    traffic_file(workload, dtype).write_text(json.dumps(rec, indent=1) + "\n")
    print(json.dumps(rec))


UNIT_ROUNDOFF = {"f32": 0.0, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        return os.cpu_count() or 1


def timed_oracle(fn, a_np, b_np, h_init, threads, seconds):
    """Run the oracle repeatedly for about ``seconds``; returns (passes, elapsed, last result)."""
    passes, ref = 0, None
    t0 = time.perf_counter()
    while True:
        ref = fn(a_np, b_np, h_init=h_init, threads=threads)
        passes += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= seconds:
            return passes, elapsed, ref


def cpu_baseline(a_np, b_np, h_last, seconds: float, single_seconds: float, shape, storage="f32", reverse=False,
                 h_init=None, a_ahead=False):
    import oracle

    if a_ahead:
        # the oracle's reverse scan over the decays taken one time step ahead;
        # the first step's decay multiplies the initial state: 1 (unused without one)
        shifted = np.empty_like(a_np)
        shifted[:, :-1] = a_np[:, 1:]
        shifted[:, -1] = 1.0
        a_np = shifted

    threads = oracle.default_threads()
    fn = oracle.linrec_oracle_rev_f64 if reverse else oracle.linrec_oracle_f64
    n = a_np.size
    passes, elapsed, ref = timed_oracle(fn, a_np, b_np, h_init, threads, seconds)
    gbs = 12.0 * n * passes / elapsed / 1e9
    # the storage type's bar: 1e-4 * (1 + |ref|), plus one rounding to a 16-bit type
    e = 1e-4 * (1.0 + np.abs(ref))
    bar = e + UNIT_ROUNDOFF[storage] * (np.abs(ref) + e)
    ratio = np.abs(h_last.astype(np.float64) - ref) / bar
    B, L, D = shape
    out = {
        "value": round(gbs, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{passes} full passes of the B={B} L={L} D={D} workload in {elapsed:.1f} s on {threads} threads "
                  f"(float64 sequential loop, 12 B/element basis)",
        "elements_per_s": round(n * passes / elapsed, 1),
        "host_cores": host_cores(),
        "cpu_model": cpu_model(),
        "gpu_check_max_bar_ratio": float(ratio.max()),
        "gpu_check_bar": "1e-4*(1+|ref|)" + ("" if storage == "f32" else f" plus one {storage} rounding"),
    }
    if single_seconds > 0:
        p1, e1, _ = timed_oracle(fn, a_np, b_np, h_init, 1, single_seconds)
        out["single_thread"] = {
            "value": round(12.0 * n * p1 / e1 / 1e9, 3),
            "unit": "GB/s",
            "elements_per_s": round(n * p1 / e1, 1),
            "sample": f"{p1} full passes in {e1:.1f} s on 1 thread",
        }
    return out


def stats_us(samples):
    x = np.asarray(samples, dtype=np.float64)
    return {"mean": round(float(x.mean()), 3), "median": round(float(np.median(x)), 3),
            "p10": round(float(np.percentile(x, 10)), 3), "p90": round(float(np.percentile(x, 90)), 3),
            "n": int(x.size)}


def region_mean_us(torch, launch, count: int, stream, first: int = 0) -> float:
    """Mean launch time (us) of ``count`` back-to-back calls ``launch(k)`` (k = first, first+1, ...)
    bracketed by one event pair on ``stream``."""
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s_ev.record(stream)
    for k in range(first, first + count):
        launch(k)
    e_ev.record(stream)
    torch.cuda.synchronize()
    return s_ev.elapsed_time(e_ev) * 1e3 / count


def measure_ceiling(torch, xs, ys, zs, rows: int, stream, warmup=3, reps=10, only=None):
    """Best mean launch time (us) of the read-2-write-1 stream over the given buffers (any storage,
    reinterpreted as float32) for each walk order; returns {order: {...}}.  ``only`` = (R, U, G)
    restricts the sweep to one walk and launch shape."""
    out = {}
    orders = (("contiguous", 1), ("scan_order", rows))
    if only is not None:
        orders = (("contiguous" if only[0] == 1 else "scan_order", only[0]),)
    for order, r in orders:
        best = sweep_walk(torch, xs, ys, zs, r, stream, warmup, reps,
                          (1, 2, 4) if only is None else (only[1],), (1, 2, 4, 8) if only is None else (only[2],))
        if best is not None:
            out[order] = best
    return out


def sweep_walk(torch, xs, ys, zs, r, stream, warmup, reps, unrolls, groups):
    """Best mean launch time of the stream walking r row streams, over the given launch shapes."""
    from linear_recurrence_scan_linrec_amd import stream_ceiling as sc

    flat = lambda t: t.reshape(-1).view(torch.float32)  # noqa: E731
    X, Y, Z = [flat(t) for t in xs], [flat(t) for t in ys], [flat(t) for t in zs]
    n = X[0].numel()
    best = None
    for unroll in unrolls:
        if n % (r * 256 * unroll) != 0:
            continue
        for gpc in groups:
            def launch(k, unroll=unroll, gpc=gpc):
                sc.stream_r2w1(X[k % len(X)], Y[k % len(X)], Z[k % len(X)], r, unroll, gpc, stream)
            for k in range(warmup):
                launch(k)
            us = region_mean_us(torch, launch, reps, stream, first=warmup)
            if best is None or us < best["us"]:
                best = {"us": round(us, 3), "rows": r, "unroll": unroll, "groups_per_cu": gpc}
    return best


def measure_tile_walk(torch, xs, ys, zs, shape, walks, stream, warmup=3, reps=10):
    """Mean launch time (us) of the read-2-write-1 stream in each tile walk (lanes, waves, rows per
    lane) over the given fp32 (B, L, D) buffers; returns a list of {...}."""
    from linear_recurrence_scan_linrec_amd import stream_ceiling as sc

    B, L, D = shape
    out = []
    for lanes, waves, t in walks:
        def launch(k, lanes=lanes, waves=waves, t=t):
            j = k % len(xs)
            sc.column_walk(xs[j], ys[j], zs[j], B, L, D, lanes, waves, t, stream)
        for k in range(warmup):
            launch(k)
        us = region_mean_us(torch, launch, reps, stream, first=warmup)
        out.append({"us": round(us, 3), "lanes": lanes, "waves": waves, "steps_per_lane": t})
    return out


def stream_rows(torch, xs, ys, zs, rows_list, stream, workload, nbytes):
    """The read-2-write-1 stream over the same buffers for each number of concurrent row streams:
    best mean launch time over unroll x groups per CU (the ceiling's own sweep)."""
    out = {"kind": "stream_rows", "workload": workload, "bytes_per_launch": nbytes, "rows": {}}
    for r in rows_list:
        b = sweep_walk(torch, xs, ys, zs, r, stream, 3, 10, (1, 2, 4), (1, 2, 4, 8))
        if b is not None:
            out["rows"][str(r)] = dict(b, gbs=round(nbytes / (b["us"] * 1e-6) / 1e9, 1))
    return out


def main():
    args = parse_args()
    if args.traffic_from:
        traffic_from(args.traffic_from[0], args.traffic_from[1], args.workload, args.dtype)
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
    if args.a_ahead and not args.reverse:
        print("--a-ahead applies to the reverse scan: add --reverse", file=sys.stderr)
        sys.exit(2)
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
    if args.stream_rows:
        print(json.dumps(stream_rows(torch, a_sets, b_sets, h_sets, [int(r) for r in args.stream_rows.split(",")],
                                     stream, args.workload, 3 * elem * n)))
        return
    plan = (lr.linrec_scan_plan(w.B, w.L, w.D) if plain else
            lr.plan_for(a_sets[0], b_sets[0], h_sets[0], h_init=h0, h_final=hf, reverse=args.reverse,
                        a_ahead=args.a_ahead))

    def step(k):
        if plain:
            lr.linrec_scan(a_sets[k], b_sets[k], h_sets[k], stream=stream)
        else:
            lr.linrec_scan(a_sets[k], b_sets[k], h_sets[k], stream=stream, h_init=h0, h_final=hf,
                           reverse=args.reverse, a_ahead=args.a_ahead)

    for i in range(args.warmup):
        step(i % sets)
    torch.cuda.synchronize()

    # the timed region: exactly --steps launches back to back, bracketed by one
    # event pair on the launch stream and by device synchronisation
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
    # the last output, taken before anything else writes the output buffers
    h_last = None if args.no_cpu_baseline else h_sets[last].float().cpu().numpy()
    launch_mean = start.elapsed_time(end) * 1e3 / args.steps
    launch = {"mean": round(launch_mean, 3)}
    if args.regions > 0:
        means = [region_mean_us(torch, lambda k: step(k % sets), 10, stream, first=10 * r) for r in range(args.regions)]
        spread = stats_us(means)
        launch.update(median=spread["median"], p10=spread["p10"], p90=spread["p90"],
                      spread_of="means of %d further regions of 10 back-to-back launches" % args.regions)

    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (wall / args.steps) / 1e9
    achieved = step_bytes / (launch_mean * 1e-6) / 1e9

    storage_name = {"f32": "fp32", "bf16": "bf16", "f16": "fp16"}[args.dtype]
    variant = "" if plain else " (linrec_scan_ex" + "".join(
        ", " + x for x in ("reverse time" if args.reverse else "",
                           "decays one step ahead" if args.a_ahead else "",
                           "initial and final state" if args.state else "")
        if x) + ")"
    headline = args.workload == li.HEADLINE and plain
    desc = w.describe(storage_name + ("" if args.dtype == "f32" else " storage, fp32 arithmetic"))
    out = {
        "metric": METRIC if headline else f"achieved HBM GB/s, linrec_scan {desc}{variant}",
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
            "workload": f"{args.workload}: {desc}{variant}",
            "B": w.B, "L": w.L, "D": w.D, "seed": seed,
            "storage": args.dtype, "arithmetic": "fp32 (fp64 products of decays on the carry path)",
            "reverse": args.reverse, "a_ahead": args.a_ahead, "state": args.state,
            "algorithmic_bytes_per_step": step_bytes,
            "buffer_sets": sets,
            "plan": plan,
        },
        "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        "elements_per_s": round(n / (wall / args.steps), 1),
        "launch_us": launch,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(args.workload, args.dtype) if not (args.reverse or args.state) else None,
        },
        "ceiling_gbs": None,
        "frac_of_ceiling": None,
        "ceiling": None,
        "cpu_baseline": None,
    }
    if not args.no_ceiling:
        only = tuple(int(x) for x in args.ceiling_shape.split(",")) if args.ceiling_shape else None
        ceil = measure_ceiling(torch, a_sets, b_sets, h_sets, w.B, stream, only=only)
        for v in ceil.values():
            v["gbs"] = round(3 * elem * n / (v["us"] * 1e-6) / 1e9, 1)
        out["ceiling"] = dict(ceil, kind="read-2-write-1 stream z = x + y (libstream_ceiling.so) over the same "
                                          "buffers; best mean launch time over unroll x groups_per_cu")
        if "contiguous" in ceil:
            out["ceiling_gbs"] = ceil["contiguous"]["gbs"]
            out["frac_of_ceiling"] = round(achieved / ceil["contiguous"]["gbs"], 4) if not args.state else None
        walks = ([tuple(int(v) for v in x.split(",")) for x in args.walk_shapes.split(";")] if args.walk_shapes else
                 [(plan["lanes_per_row"], plan["waves"], plan["steps_per_lane"])])
        # the plan's own walk when it is one sequence per workgroup: a local carry whose grid is
        # the sequences themselves (from the CU count up to twice it)
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        lanes = plan["lanes_per_row"]
        nseq = w.B * (w.D // (4 * lanes)) if lanes >= 8 and w.D % (4 * lanes) == 0 else 0
        own = (args.dtype == "f32" and plan["mode"] in (0, 2) and plan["vec"] == 4 and cus <= nseq < 2 * cus
               and plan["waves"] in (1, 2, 4, 8) and plan["steps_per_lane"] in (4, 8))
        if only is None and args.dtype == "f32" and (own or args.walk_shapes):
            tw = measure_tile_walk(torch, a_sets, b_sets, h_sets, (w.B, w.L, w.D), walks, stream)
            for v in tw:
                v["gbs"] = round(3 * elem * n / (v["us"] * 1e-6) / 1e9, 1)
                v["frac_scan"] = round(achieved / v["gbs"], 4) if not args.state else None
            out["ceiling"]["tile_walk"] = tw[0] if len(tw) == 1 else tw
    if args.cold > 0:
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        cold, warm = [], []
        for i in range(args.cold):
            for evict, into in ((True, cold), (False, warm)):
                if evict:
                    flush.fill_(float(i))
                into.append(region_mean_us(torch, lambda k: step(k % sets), 1, stream, first=i))
        del flush
        out["single_launch_us"] = {"cold": stats_us(cold), "warm": stats_us(warm),
                                   "note": "one event pair per launch (adds its own overhead to both)"}
    if args.calibration_copy:
        src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.calibration_copy):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        # the oracle on the values the GPU consumed (16-bit inputs widen exactly)
        out["cpu_baseline"] = cpu_baseline(a_host.float().numpy(), b_host.float().numpy(), h_last, args.cpu_seconds,
                                           args.cpu_single_seconds, (w.B, w.L, w.D), storage=args.dtype,
                                           reverse=args.reverse, h_init=h0_np, a_ahead=args.a_ahead)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
