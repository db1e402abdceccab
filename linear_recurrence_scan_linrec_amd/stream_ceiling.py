"""ctypes binding of ``libstream_ceiling.so`` (``include/linrec_stream.h``): the read-two-write-one
stream z = x + y that bench.py measures the scan against.  Argument marshalling only; importing
raises ``ImportError`` when the library has not been built."""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch  # noqa: F401  (loads the HIP runtime the library links against first)

LIBRARY = Path(__file__).resolve().parent / "lib" / "libstream_ceiling.so"
EXPORTED = ("linrec_stream_r2w1", "linrec_stream_column_walk", "linrec_stream_last_error")


def _load() -> ctypes.CDLL:
    if not LIBRARY.exists():
        raise ImportError(f"{LIBRARY} is missing: build it with `python -m linear_recurrence_scan_linrec_amd.build`")
    lib = ctypes.CDLL(str(LIBRARY))
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.linrec_stream_r2w1.restype = ctypes.c_int
    lib.linrec_stream_r2w1.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp]
    lib.linrec_stream_column_walk.restype = ctypes.c_int
    lib.linrec_stream_column_walk.argtypes = [vp, vp, vp, i64, i64, i64, i32, i32, i32, vp]
    lib.linrec_stream_last_error.restype = ctypes.c_char_p
    lib.linrec_stream_last_error.argtypes = []
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def stream_r2w1(x, y, z, rows: int = 1, unroll: int = 4, groups_per_cu: int = 2, stream=None) -> None:
    """Enqueue z = x + y over the float32 elements of three same-sized CUDA tensors (any storage
    reinterpreted as float32 by the caller) on ``stream`` (default: the current stream)."""
    n = x.numel()
    if y.numel() != n or z.numel() != n:
        raise ValueError("x, y and z must have the same number of elements")
    s = (stream if stream is not None else torch.cuda.current_stream()).cuda_stream
    status = _lib.linrec_stream_r2w1(x.data_ptr(), y.data_ptr(), z.data_ptr(), n, rows, unroll, groups_per_cu, s)
    if status != 0:
        raise RuntimeError(f"linrec_stream_r2w1: {_lib.linrec_stream_last_error().decode()}")


def column_walk(x, y, z, B: int, L: int, D: int, lanes: int, waves: int, steps_per_lane: int, stream=None) -> None:
    """Enqueue z = x + y over three contiguous (B, L, D) float32 CUDA tensors in the walk of the
    scan's local-carry plans (``linrec_stream_column_walk``) on ``stream``."""
    for t in (x, y, z):
        if t.numel() != B * L * D:
            raise ValueError("x, y and z must hold B * L * D elements")
    s = (stream if stream is not None else torch.cuda.current_stream()).cuda_stream
    status = _lib.linrec_stream_column_walk(x.data_ptr(), y.data_ptr(), z.data_ptr(), B, L, D, lanes, waves,
                                            steps_per_lane, s)
    if status != 0:
        raise RuntimeError(f"linrec_stream_column_walk: {_lib.linrec_stream_last_error().decode()}")
