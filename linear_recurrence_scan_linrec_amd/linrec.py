"""ctypes binding of ``liblinrec.so`` (the C ABI in ``include/linrec.h``).

Argument marshalling only: every step of the scan runs in the library's HIP
kernels.  PyTorch provides device memory and streams.  Importing this module
raises ``ImportError`` when the library has not been built
(``python -m linear_recurrence_scan_linrec_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

# PyTorch's ROCm wheel carries its own HIP runtime (soname libamdhip64.so.7) and
# loads it by file name.  Importing torch first lets the library's dependency on
# that soname resolve to the runtime already in the process; loading the library
# first would leave two HIP runtimes in one process, and the second one sees no
# device.
import torch  # noqa: F401

LIBRARY = Path(__file__).resolve().parent / "lib" / "liblinrec.so"

LINREC_OK = 0
LINREC_ERR_INVALID_ARGUMENT = 1
LINREC_ERR_OVERLAP = 2
LINREC_ERR_HIP = 3
LINREC_ERR_OUT_OF_MEMORY = 4

# Every function include/linrec.h declares.
EXPORTED = (
    "linrec_scan",
    "linrec_scan_plan",
    "linrec_status_string",
    "linrec_last_error_message",
    "linrec_device_timeouts",
    "linrec_release",
)


class linrec_plan(ctypes.Structure):
    _fields_ = [
        ("vec", ctypes.c_int32),
        ("steps_per_lane", ctypes.c_int32),
        ("waves", ctypes.c_int32),
        ("lanes_per_row", ctypes.c_int32),
        ("steps_per_tile", ctypes.c_int64),
        ("chunks", ctypes.c_int64),
        ("tiles", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_size_t),
        ("mode", ctypes.c_int32),
    ]


class LinrecError(RuntimeError):
    """A linrec_* call returned a status other than LINREC_OK."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{linrec_status_string(status)} ({status}): {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not LIBRARY.exists():
        raise ImportError(f"{LIBRARY} is missing: build it with "
                          "`python -m linear_recurrence_scan_linrec_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(str(LIBRARY))
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.linrec_scan.restype = ctypes.c_int
    lib.linrec_scan.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.linrec_scan_plan.restype = ctypes.c_int
    lib.linrec_scan_plan.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(linrec_plan)]
    lib.linrec_status_string.restype = ctypes.c_char_p
    lib.linrec_status_string.argtypes = [ctypes.c_int]
    lib.linrec_last_error_message.restype = ctypes.c_char_p
    lib.linrec_last_error_message.argtypes = []
    lib.linrec_device_timeouts.restype = ctypes.c_int
    lib.linrec_device_timeouts.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    lib.linrec_release.restype = None
    lib.linrec_release.argtypes = []
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    """The loaded ``liblinrec.so``."""
    return _lib


def linrec_status_string(status: int) -> str:
    return _lib.linrec_status_string(int(status)).decode()


def linrec_last_error_message() -> str:
    return _lib.linrec_last_error_message().decode()


def _check(status: int) -> None:
    if status != LINREC_OK:
        raise LinrecError(status, linrec_last_error_message())


def linrec_scan_raw(a_ptr: int, b_ptr: int, h_ptr: int, B: int, L: int, D: int, stream_ptr: int = 0) -> int:
    """Direct C-ABI call with raw device pointers; returns the status code."""
    return _lib.linrec_scan(a_ptr, b_ptr, h_ptr, B, L, D, stream_ptr)


def linrec_scan(a, b, h=None, stream=None):
    """h[i,0,d] = b[i,0,d], h[i,t,d] = a[i,t,d]*h[i,t-1,d] + b[i,t,d] on the GPU.

    ``a`` and ``b`` are contiguous fp32 CUDA tensors of shape (B, L, D) on one
    device; ``h`` (optional) receives the result and is allocated when omitted.
    The call is enqueued on ``stream`` (a ``torch.cuda.Stream``; default: the
    current stream of a's device) and returns without synchronising.
    """
    for name, t in (("a", a), ("b", b)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.float32 or not t.is_cuda or t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 CUDA tensor of shape (B, L, D)")
    if a.shape != b.shape or a.device != b.device:
        raise ValueError("a and b must have one shape and one device")
    if h is None:
        h = torch.empty_like(a)
    elif (h.shape != a.shape or h.dtype != torch.float32 or h.device != a.device
          or not h.is_contiguous()):
        raise ValueError("h must be a contiguous float32 tensor shaped and placed like a")
    B, L, D = a.shape
    if a.device.index == torch.cuda.current_device():
        s = torch.cuda.current_stream() if stream is None else stream
        _check(_lib.linrec_scan(a.data_ptr(), b.data_ptr(), h.data_ptr(), B, L, D, s.cuda_stream))
        return h
    with torch.cuda.device(a.device):   # the library works on the current HIP device
        s = torch.cuda.current_stream(a.device) if stream is None else stream
        _check(_lib.linrec_scan(a.data_ptr(), b.data_ptr(), h.data_ptr(), B, L, D, s.cuda_stream))
    return h


def linrec_scan_plan(B: int, L: int, D: int, aligned16: bool = True) -> dict:
    """The tile, launch size and workspace linrec_scan would use for (B, L, D)."""
    plan = linrec_plan()
    _check(_lib.linrec_scan_plan(B, L, D, int(bool(aligned16)), ctypes.byref(plan)))
    return {name: getattr(plan, name) for name, _ in linrec_plan._fields_}


def linrec_device_timeouts() -> int:
    """Tiles on the current device that gave up waiting for their carry (synchronises)."""
    count = ctypes.c_uint64(0)
    _check(_lib.linrec_device_timeouts(ctypes.byref(count)))
    return int(count.value)


def linrec_release() -> None:
    """Free the library's per-device workspaces (no scan may still be running)."""
    _lib.linrec_release()
