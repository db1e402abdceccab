"""Build the gfx950 shared library ``liblinrec.so`` in-tree with hipcc.

``python -m linear_recurrence_scan_linrec_amd.build`` compiles
``csrc/linrec.hip`` (kernels and the C ABI of ``include/linrec.h``) into
``linear_recurrence_scan_linrec_amd/lib/liblinrec.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PACKAGE = Path(__file__).resolve().parent
ROOT = PACKAGE.parent
INCLUDE = ROOT / "include"
SOURCES = [PACKAGE / "csrc" / "linrec.hip"]
DEPENDS = SOURCES + [PACKAGE / "csrc" / "scan_kernel.hpp", INCLUDE / "linrec.h"]
LIBRARY = PACKAGE / "lib" / "liblinrec.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
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


def build(output: Path = LIBRARY, extra_flags=(), verbose: bool = False) -> Path:
    """Compile the library; always recompiles."""
    output.parent.mkdir(parents=True, exist_ok=True)
    tmp = output.with_suffix(".so.tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, f"-I{INCLUDE}", *map(str, SOURCES), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"hipcc failed with exit code {proc.returncode}")
    os.replace(tmp, output)
    return output


def is_stale(output: Path = LIBRARY) -> bool:
    if not output.exists():
        return True
    built = output.stat().st_mtime
    return any(p.stat().st_mtime > built for p in DEPENDS)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
