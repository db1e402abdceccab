"""float64 CPU oracle for the channel-wise linear recurrence.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import or
call this package.  It shares no code with the HIP path and the HIP path never
calls it.

The arithmetic lives in ``linrec_oracle.c`` (the plain sequential definition
h_0 = b_0, h_t = a_t * h_{t-1} + b_t in float64; see the header there for the
passages it follows).  This module only builds and loads that C file and
marshals numpy arrays to it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
SOURCE = _HERE / "linrec_oracle.c"
LIBRARY = _HERE / "liblinrec_oracle.so"

# Portable flags: the library is built in one container and may run on another
# host CPU, so no -march=native.  -ffp-contract=off keeps multiply and add
# separately rounded in every iteration.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off"]

_lib = None


def build(source: Path = SOURCE, output: Path = LIBRARY, extra_flags=()) -> Path:
    """Compile ``source`` with gcc into the shared library ``output``."""
    cmd = ["gcc", *CFLAGS, *extra_flags, str(source), "-o", str(output)]
    subprocess.run(cmd, check=True)
    return output


def load_library(path: Path | str) -> ctypes.CDLL:
    """Load an oracle shared library and declare its entry points."""
    lib = ctypes.CDLL(str(path))
    for fn in (lib.linrec_oracle_f64, lib.linrec_oracle_rev_f64):
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    return lib


def _library() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not LIBRARY.exists() or LIBRARY.stat().st_mtime < SOURCE.stat().st_mtime:
            build()
        _lib = load_library(LIBRARY)
    return _lib


def default_threads() -> int:
    """Host threads the oracle uses by default: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def call_library(lib: ctypes.CDLL, a: np.ndarray, b: np.ndarray, h_init=None, threads=None,
                 reverse: bool = False) -> np.ndarray:
    """Run ``lib``'s oracle (the reverse-time form if ``reverse``) on fp32 (B, L, D) arrays;
    returns float64 (B, L, D)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    if a.ndim != 3 or a.shape != b.shape:
        raise ValueError(f"a and b must be (B, L, D) arrays of one shape, got {a.shape} and {b.shape}")
    B, L, D = a.shape
    hi = None
    if h_init is not None:
        hi = np.ascontiguousarray(h_init, dtype=np.float64)
        if hi.shape != (B, D):
            raise ValueError(f"h_init must be (B, D) = {(B, D)}, got {hi.shape}")
    h = np.empty((B, L, D), dtype=np.float64)
    fn = lib.linrec_oracle_rev_f64 if reverse else lib.linrec_oracle_f64
    rc = fn(a.ctypes.data, b.ctypes.data,
                               None if hi is None else hi.ctypes.data,
                               h.ctypes.data, B, L, D,
                               default_threads() if threads is None else int(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return h


def linrec_oracle_f64(a: np.ndarray, b: np.ndarray, h_init=None, threads=None) -> np.ndarray:
    """float64 reference h for fp32 inputs a, b of shape (B, L, D).

    ``h_init`` (B, D), when given, is the state before t = 0, so that
    h_0 = a_0 * h_init + b_0; without it the state is zero and h_0 = b_0.
    """
    return call_library(_library(), a, b, h_init=h_init, threads=threads)


def linrec_oracle_rev_f64(a: np.ndarray, b: np.ndarray, h_init=None, threads=None) -> np.ndarray:
    """float64 reference of the reverse-time recurrence h_t = a_t * h_{t+1} + b_t for fp32 inputs
    of shape (B, L, D), run from t = L-1 down to 0.

    ``h_init`` (B, D), when given, is the state after the last step, so that
    h_{L-1} = a_{L-1} * h_init + b_{L-1}; without it the state is zero and h_{L-1} = b_{L-1}.
    """
    return call_library(_library(), a, b, h_init=h_init, threads=threads, reverse=True)
