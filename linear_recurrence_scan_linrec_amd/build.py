"""Build the gfx950 shared libraries in-tree with hipcc.

``python -m linear_recurrence_scan_linrec_amd.build`` compiles the host side of
the C ABI of ``include/linrec.h`` (``csrc/linrec.hip``) and the kernel instances
for each storage type (``csrc/kernels_{f32,bf16,f16}.hip``) in parallel, then
links them into ``linear_recurrence_scan_linrec_amd/lib/liblinrec.so``.  It also
builds ``lib/libstream_ceiling.so`` (``include/linrec_stream.h``,
``csrc/stream_ceiling.hip``): the read-two-write-one stream that bench.py
measures the scan against.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PACKAGE = Path(__file__).resolve().parent
ROOT = PACKAGE.parent
INCLUDE = ROOT / "include"
CSRC = PACKAGE / "csrc"
SOURCES = [CSRC / "linrec.hip", CSRC / "kernels_f32.hip", CSRC / "kernels_bf16.hip", CSRC / "kernels_f16.hip"]
DEPENDS = SOURCES + [CSRC / "scan_kernel.hpp", CSRC / "call_epoch.hpp", CSRC / "launch.hpp", CSRC / "instances.hpp",
                     INCLUDE / "linrec.h"]
LIBRARY = PACKAGE / "lib" / "liblinrec.so"
STREAM_SOURCES = [CSRC / "stream_ceiling.hip"]
STREAM_LIBRARY = PACKAGE / "lib" / "libstream_ceiling.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep hipcc from forming packed-fp32 instructions (the host pass warns about
    # the unknown feature; that is expected)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    found = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(found).exists():
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build liblinrec.so")
    return found


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"hipcc failed with exit code {proc.returncode}: {' '.join(cmd[-3:])}")


def _link(sources, output: Path, extra_flags, verbose: bool, pool) -> Path:
    output.parent.mkdir(parents=True, exist_ok=True)
    tmp = output.with_suffix(".so.tmp")
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="linrec_build_") as work:
        objects = [Path(work) / (src.stem + ".o") for src in sources]
        cmds = [[cc, *HIPCC_FLAGS, *extra_flags, f"-I{INCLUDE}", f"-I{CSRC}", "-c", str(src), "-o", str(obj)]
                for src, obj in zip(sources, objects)]
        for f in [pool.submit(_run, cmd, verbose) for cmd in cmds]:
            f.result()
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objects), "-o", str(tmp)], verbose)
    os.replace(tmp, output)
    return output


def build(output: Path = LIBRARY, extra_flags=(), verbose: bool = False, stream_output: Path = STREAM_LIBRARY) -> Path:
    """Compile the scan library and the streaming-ceiling library; always recompiles.  Returns the
    scan library's path."""
    jobs = max(1, min(len(SOURCES) + len(STREAM_SOURCES), os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        stream = pool.submit(_link, STREAM_SOURCES, stream_output, extra_flags, verbose, pool)
        _link(SOURCES, output, extra_flags, verbose, pool)
        stream.result()
    return output


def is_stale(output: Path = LIBRARY) -> bool:
    if not output.exists():
        return True
    built = output.stat().st_mtime
    return any(p.stat().st_mtime > built for p in DEPENDS)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
