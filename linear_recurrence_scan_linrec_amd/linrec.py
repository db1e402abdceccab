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
    "linrec_scan_ex",
    "linrec_scan_ex_plan",
    "linrec_status_string",
    "linrec_last_error_message",
    "linrec_device_timeouts",
    "linrec_release",
    "linrec_scan_ws",
    "linrec_scan_ex_ws",
    "linrec_scan_workspace_bytes",
    "linrec_scan_ex_workspace_bytes",
    "linrec_scan_ex_noalloc",
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


class linrec_operand(ctypes.Structure):
    _fields_ = [
        ("ptr", ctypes.c_void_p),
        ("stride_b", ctypes.c_int64),
        ("stride_l", ctypes.c_int64),
    ]


class linrec_scan_desc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64),
        ("L", ctypes.c_int64),
        ("D", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("reverse", ctypes.c_int32),
        ("a", linrec_operand),
        ("b", linrec_operand),
        ("h", linrec_operand),
        ("h_init", ctypes.c_void_p),
        ("h_final", ctypes.c_void_p),
    ]


LINREC_F32, LINREC_BF16, LINREC_F16 = 0, 1, 2
DTYPES = {torch.float32: LINREC_F32, torch.bfloat16: LINREC_BF16, torch.float16: LINREC_F16}


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
    lib.linrec_scan_ex.restype = ctypes.c_int
    lib.linrec_scan_ex.argtypes = [ctypes.POINTER(linrec_scan_desc), vp]
    lib.linrec_scan_ex_plan.restype = ctypes.c_int
    lib.linrec_scan_ex_plan.argtypes = [ctypes.POINTER(linrec_scan_desc), ctypes.POINTER(linrec_plan)]
    lib.linrec_status_string.restype = ctypes.c_char_p
    lib.linrec_status_string.argtypes = [ctypes.c_int]
    lib.linrec_last_error_message.restype = ctypes.c_char_p
    lib.linrec_last_error_message.argtypes = []
    lib.linrec_device_timeouts.restype = ctypes.c_int
    lib.linrec_device_timeouts.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    lib.linrec_release.restype = None
    lib.linrec_release.argtypes = []
    lib.linrec_scan_ws.restype = ctypes.c_int
    lib.linrec_scan_ws.argtypes = [vp, vp, vp, i64, i64, i64, vp, ctypes.c_size_t, vp]
    lib.linrec_scan_ex_ws.restype = ctypes.c_int
    lib.linrec_scan_ex_ws.argtypes = [ctypes.POINTER(linrec_scan_desc), vp, ctypes.c_size_t, vp]
    lib.linrec_scan_workspace_bytes.restype = ctypes.c_size_t
    lib.linrec_scan_workspace_bytes.argtypes = [i64, i64, i64]
    lib.linrec_scan_ex_workspace_bytes.restype = ctypes.c_int
    lib.linrec_scan_ex_workspace_bytes.argtypes = [ctypes.POINTER(linrec_scan_desc), ctypes.POINTER(ctypes.c_size_t)]
    lib.linrec_scan_ex_noalloc.restype = ctypes.c_int
    lib.linrec_scan_ex_noalloc.argtypes = [ctypes.POINTER(linrec_scan_desc), vp]
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


def _operand(t) -> linrec_operand:
    return linrec_operand(t.data_ptr(), t.stride(0), t.stride(1))


def _check_operand(name, t, like=None):
    """Checks one (B, L, D) operand; with `like` (a's size, dtype and device index), that it
    matches.  Returns the operand's (size, dtype, device index)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    size = t.size()
    if not t.is_cuda or len(size) != 3:
        raise ValueError(f"{name} must be a CUDA tensor of shape (B, L, D)")
    dtype = t.dtype
    if dtype not in DTYPES:
        raise ValueError(f"{name} must be float32, bfloat16 or float16, not {dtype}")
    if size[2] > 1 and t.stride()[2] != 1:
        raise ValueError(f"{name} must have unit stride along D (the last dimension)")
    sig = (size, dtype, t.get_device())
    if like is not None and sig != like:
        raise ValueError(f"{name} must be shaped, typed and placed like a: {tuple(like[0])} {like[1]} cuda:{like[2]}")
    return sig


def _check_state(name, t, B, D, device):
    if t is None:
        return
    if (not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda or tuple(t.shape) != (B, D)
            or t.device != device or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous float32 CUDA tensor of shape (B, D) = {(B, D)} on {device}")


def make_desc(a, b, h, h_init=None, h_final=None, reverse=False, a_ahead=False) -> linrec_scan_desc:
    """The linrec_scan_desc for torch tensors (no checks beyond what ctypes needs); ``a_ahead``
    selects the reverse form whose decays are taken one time step ahead (``reverse`` = 2)."""
    B, L, D = a.shape
    mode = 2 if a_ahead else int(bool(reverse))
    return linrec_scan_desc(B, L, D, DTYPES[a.dtype], mode, _operand(a), _operand(b), _operand(h),
                            None if h_init is None else h_init.data_ptr(),
                            None if h_final is None else h_final.data_ptr())


# torch's raw current-stream query (one C call); the public form builds a Stream object first.
_current_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_ptr(stream, index: int) -> int:
    if stream is not None:
        return stream.cuda_stream
    if _current_raw_stream is not None:
        return _current_raw_stream(index)
    return torch.cuda.current_stream(index).cuda_stream


def _enqueue(a, b, h, h_init, h_final, reverse, a_ahead, plain, stream_ptr, workspace):
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        if plain:
            B, L, D = a.size()
            _check(_lib.linrec_scan_ws(a.data_ptr(), b.data_ptr(), h.data_ptr(), B, L, D, ws_ptr, ws_bytes,
                                       stream_ptr))
        else:
            desc = make_desc(a, b, h, h_init, h_final, reverse, a_ahead)
            _check(_lib.linrec_scan_ex_ws(ctypes.byref(desc), ws_ptr, ws_bytes, stream_ptr))
    elif plain:
        B, L, D = a.size()
        _check(_lib.linrec_scan(a.data_ptr(), b.data_ptr(), h.data_ptr(), B, L, D, stream_ptr))
    else:
        desc = make_desc(a, b, h, h_init, h_final, reverse, a_ahead)
        _check(_lib.linrec_scan_ex(ctypes.byref(desc), stream_ptr))


def linrec_scan(a, b, h=None, stream=None, *, h_init=None, h_final=None, return_final=False, reverse=False,
                a_ahead=False, workspace=None):
    """The channel-wise linear recurrence on the GPU.

    Forward (default): h[i,0,d] = a[i,0,d]*h_init[i,d] + b[i,0,d] (h_init taken as 0 when
    omitted, so h[i,0,d] = b[i,0,d]) and h[i,t,d] = a[i,t,d]*h[i,t-1,d] + b[i,t,d].
    ``reverse=True`` runs the same recurrence from t = L-1 down to 0 (h[i,t,d] uses h[i,t+1,d]).
    ``a_ahead=True`` (with ``reverse=True``) takes each decay one time step ahead:
    h[i,L-1,d] = h_init[i,d] + b[i,L-1,d] (0 for h_init when omitted) and
    h[i,t,d] = a[i,t+1,d]*h[i,t+1,d] + b[i,t,d].  With an incoming gradient g as ``b`` this is
    dLoss/db of the forward scan over ``a``, read straight from ``a`` without a shifted copy;
    a sequence taken in pieces chains through h_init = a[:, L] * (the next piece's result at
    its first step).

    ``a`` and ``b`` are CUDA tensors of shape (B, L, D), one dtype (float32, bfloat16 or
    float16), unit stride along D and any non-negative strides otherwise (views, expanded or
    time-major layouts work without copies); arithmetic is fp32.  ``h`` (optional) receives the
    result in the same dtype and is allocated contiguous when omitted.  ``h_init`` is an
    optional (B, D) float32 state before the first step; ``h_final`` an optional (B, D) float32
    tensor that receives the state after the last step (allocated when ``return_final``).
    Returns ``h``, or ``(h, h_final)`` when a final state is asked for.  The call is enqueued on
    ``stream`` (default: the current stream of a's device) and returns without synchronising.
    ``workspace`` (optional): a zero-filled CUDA tensor on a's device, 256-byte aligned, of at least
    ``workspace_bytes(...)`` bytes, used as the lookback workspace instead of the library's own
    for the stream (linrec_scan_ws / linrec_scan_ex_ws).

    Under CUDA-graph capture of the current stream (``torch.cuda.graph``), a call that needs a
    lookback workspace and is given none gets one from the graph's memory pool, zero-filled by a
    fill kernel recorded in the graph before the scan, so that every replay starts from a clean
    workspace (the library itself never allocates while a stream is captured).
    """
    if a_ahead and not reverse:
        raise ValueError("a_ahead applies to the reverse scan (reverse=True)")
    like = _check_operand("a", a)
    _check_operand("b", b, like)
    (B, L, D), dtype, index = like
    if h is None:
        h = torch.empty((B, L, D), dtype=dtype, device=a.device)
    else:
        _check_operand("h", h, like)
    want_final = return_final or h_final is not None
    if h_init is not None:
        _check_state("h_init", h_init, B, D, a.device)
    if want_final:
        if h_final is None:
            h_final = torch.empty((B, D), dtype=torch.float32, device=a.device)
        else:
            _check_state("h_final", h_final, B, D, a.device)
    plain = (dtype is torch.float32 and not reverse and h_init is None and not want_final
             and a.is_contiguous() and b.is_contiguous() and h.is_contiguous())
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or workspace.device != a.device
                                  or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous CUDA tensor on a's device")
    if workspace is None and stream is None and torch.cuda.is_current_stream_capturing():
        need = workspace_bytes(a, b, h, h_init=h_init, h_final=h_final, reverse=reverse, a_ahead=a_ahead)
        if need > 0:
            # from the capture's memory pool; torch's allocations are 512-byte aligned
            workspace = torch.zeros(need, dtype=torch.uint8, device=a.device)
    if index != torch.cuda.current_device():
        with torch.cuda.device(index):   # the library works on the current HIP device
            _enqueue(a, b, h, h_init, h_final, reverse, a_ahead, plain, _stream_ptr(stream, index), workspace)
    else:
        _enqueue(a, b, h, h_init, h_final, reverse, a_ahead, plain, _stream_ptr(stream, index), workspace)
    return (h, h_final) if want_final else h


def workspace_bytes(a, b, h=None, *, h_init=None, h_final=None, reverse=False, a_ahead=False) -> int:
    """Bytes of the lookback workspace a linrec_scan of these tensors may need on their device
    (0: none); the size a ``workspace`` argument must have."""
    desc = make_desc(a, b, a if h is None else h, h_init, h_final, reverse, a_ahead)
    out = ctypes.c_size_t(0)
    with torch.cuda.device(a.get_device()):
        _check(_lib.linrec_scan_ex_workspace_bytes(ctypes.byref(desc), ctypes.byref(out)))
    return int(out.value)


def linrec_scan_ex_raw(desc: linrec_scan_desc, stream_ptr: int = 0) -> int:
    """Direct C-ABI call of linrec_scan_ex; returns the status code."""
    return _lib.linrec_scan_ex(ctypes.byref(desc), stream_ptr)


def plan_for(a, b, h=None, *, h_init=None, h_final=None, reverse=False, a_ahead=False) -> dict:
    """The plan linrec_scan_ex would use for these tensors (host arithmetic only)."""
    desc = make_desc(a, b, a if h is None else h, h_init, h_final, reverse, a_ahead)
    plan = linrec_plan()
    _check(_lib.linrec_scan_ex_plan(ctypes.byref(desc), ctypes.byref(plan)))
    return {name: getattr(plan, name) for name, _ in linrec_plan._fields_}


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
