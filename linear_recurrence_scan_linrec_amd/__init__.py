"""MI355X (gfx950) channel-wise linear-recurrence scan.

h[i,0,d] = b[i,0,d];  h[i,t,d] = a[i,t,d] * h[i,t-1,d] + b[i,t,d]  over (B, L, D)
fp32 tensors with D contiguous, evaluated by hand-written HIP kernels behind
the C ABI in ``include/linrec.h``.  The names below are loaded from
``linear_recurrence_scan_linrec_amd.linrec`` on first use, which raises
``ImportError`` when ``lib/liblinrec.so`` has not been built.
"""
_EXPORTS = (
    "linrec_scan",
    "linrec_scan_raw",
    "linrec_scan_plan",
    "linrec_status_string",
    "linrec_last_error_message",
    "linrec_device_timeouts",
    "linrec_release",
    "LinrecError",
)

__all__ = list(_EXPORTS)


def __getattr__(name):
    if name in _EXPORTS:
        from . import linrec as _binding
        return getattr(_binding, name)
    raise AttributeError(name)
