"""Seeded random descriptors through the host-only entry points (linrec_scan_ex_plan,
linrec_scan_plan): no HIP call is made, so this runs on the CPU.  Each decision is checked
against what the header documents, with the overlap rule checked by brute force:

- every descriptor the header says is invalid (negative size or stride, unknown dtype or
  direction, a, b or h misaligned to its element size, h_init or h_final misaligned to 4 bytes,
  rows of h that overlap) is rejected with LINREC_ERR_INVALID_ARGUMENT;
- every descriptor the library accepts has pairwise disjoint rows of h (brute force over every
  (i, t) row start) and a plan whose fields agree with each other;
- a valid descriptor that is rejected all the same names one of the documented limits in its
  message: strides of h that do not nest (see linrec_scan_desc), a tile spanning 1 GiB, more
  than 2^31 - 1 tiles, or sizes that overflow.
"""
import ctypes

import numpy as np
import pytest

from linear_recurrence_scan_linrec_amd import linrec as lr

ES = {lr.LINREC_F32: 4, lr.LINREC_BF16: 2, lr.LINREC_F16: 2}
BASE = 1 << 40   # stand-in addresses: the plan entry points never dereference them


def rows_overlap(B, L, D, sb, sl):
    """True when two rows (i, t) of h share an element (brute force)."""
    starts = sorted(i * sb + t * sl for i in range(B) for t in range(L))
    return any(b_ < a_ + D for a_, b_ in zip(starts, starts[1:]))


def draw(rng):
    """A random descriptor: mostly plausible, sometimes broken in one documented way."""
    B, L, D = (int(rng.integers(0, 5)), int(rng.integers(0, 40)), int(rng.integers(0, 20)))
    if rng.random() < 0.05:
        B, L, D = [x if rng.random() < 0.7 else -int(rng.integers(1, 3)) for x in (B, L, D)]
    dtype = int(rng.choice([0, 1, 2])) if rng.random() < 0.97 else int(rng.choice([-1, 3]))
    reverse = int(rng.choice([0, 1, 2])) if rng.random() < 0.97 else int(rng.choice([-1, 3]))
    es = ES.get(dtype, 4)

    def operand(k):
        contiguous = rng.random() < 0.5
        sl = max(D, 0) if contiguous else int(rng.integers(0, 3 * max(D, 1) + 2))
        sb = max(L, 0) * sl if contiguous else int(rng.integers(0, 3 * max(L * max(D, 1), 1) + 2))
        if rng.random() < 0.03:
            sl = -int(rng.integers(1, 4))
        if rng.random() < 0.03:
            sb = -int(rng.integers(1, 4))
        misalign = int(rng.integers(1, es)) if (es > 1 and rng.random() < 0.05) else 0
        vec_misalign = int(rng.choice([0, es, 2 * es])) if rng.random() < 0.3 else 0
        ptr = BASE + (k << 32) + vec_misalign + misalign
        return lr.linrec_operand(ptr, sb, sl)

    d = lr.linrec_scan_desc()
    d.B, d.L, d.D, d.dtype, d.reverse = B, L, D, dtype, reverse
    d.a, d.b, d.h = operand(0), operand(1), operand(2)
    d.h_init = None if rng.random() < 0.6 else BASE + (3 << 32) + (int(rng.integers(1, 4)) if rng.random() < 0.1 else 0)
    d.h_final = None if rng.random() < 0.6 else BASE + (4 << 32) + (int(rng.integers(1, 4)) if rng.random() < 0.1 else 0)
    return d


def documented_invalid(d):
    """The reason the header gives for rejecting d, or None."""
    if min(d.B, d.L, d.D) < 0:
        return "negative size"
    if d.dtype not in ES:
        return "dtype"
    if d.reverse not in (0, 1, 2):
        return "reverse"
    ops = (d.a, d.b, d.h)
    if any(o.stride_b < 0 or o.stride_l < 0 for o in ops):
        return "negative stride"
    es = ES[d.dtype]
    if any(o.ptr % es for o in ops):
        return "operand alignment"
    if (d.h_init or 0) % 4 or (d.h_final or 0) % 4:
        return "state alignment"
    if d.B * d.L * d.D > 0:
        sb = d.h.stride_b if d.B > 1 else 0
        sl = d.h.stride_l if d.L > 1 else d.D
        if rows_overlap(d.B, d.L, d.D, sb, sl):
            return "rows of h overlap"
    return None


def test_random_descriptors_follow_the_documented_rules():
    rng = np.random.default_rng(20261202)
    lib = lr.library()
    counts = {"accepted": 0, "documented": 0, "limit": 0}
    for case in range(4000):
        d = draw(rng)
        plan = lr.linrec_plan()
        status = lib.linrec_scan_ex_plan(ctypes.byref(d), ctypes.byref(plan))
        msg = lr.linrec_last_error_message()
        why = documented_invalid(d)
        label = (f"case {case}: B={d.B} L={d.L} D={d.D} dtype={d.dtype} reverse={d.reverse} "
                 f"a=({d.a.stride_b},{d.a.stride_l}) h=({d.h.stride_b},{d.h.stride_l}) -> {status} {msg!r}")
        if why is not None:
            assert status == lr.LINREC_ERR_INVALID_ARGUMENT, f"{label}; expected a rejection: {why}"
            counts["documented"] += 1
            continue
        if status != lr.LINREC_OK:
            assert status == lr.LINREC_ERR_INVALID_ARGUMENT, label
            assert any(k in msg for k in ("overlap one another", "1 GiB", "2^31", "63 bits", "2^63")), label
            counts["limit"] += 1
            continue
        counts["accepted"] += 1
        empty = d.B * d.L * d.D == 0
        assert (plan.tiles == 0) == empty, label
        if not empty:
            assert plan.steps_per_tile == plan.waves * (64 // plan.lanes_per_row) * plan.steps_per_lane, label
            assert plan.chunks == -(-d.L // plan.steps_per_tile), label
            assert plan.tiles % plan.chunks == 0, label
            assert (plan.workspace_bytes > 0) == (plan.chunks > 1), label
            assert plan.vec in (1, 4) and plan.mode in (0, 1, 2), label
    # the draw exercises every branch
    assert min(counts.values()) > 20, counts


@pytest.mark.parametrize("seed", [1, 2])
def test_random_plain_shapes(seed):
    rng = np.random.default_rng(seed)
    lib = lr.library()
    for _ in range(1000):
        B, L, D = (int(x) for x in rng.integers(-2, 300, size=3))
        if rng.random() < 0.1:
            B, L, D = (int(x) for x in rng.integers(0, 1 << 21, size=3))
        plan = lr.linrec_plan()
        status = lib.linrec_scan_plan(B, L, D, int(rng.integers(0, 2)), ctypes.byref(plan))
        if min(B, L, D) < 0:
            assert status == lr.LINREC_ERR_INVALID_ARGUMENT
        elif B * L * D * 8 > (1 << 63) - 1:
            assert status == lr.LINREC_ERR_INVALID_ARGUMENT and "63 bits" in lr.linrec_last_error_message()
        elif status == lr.LINREC_OK:
            assert (plan.tiles == 0) == (B * L * D == 0)
        else:
            assert "2^31" in lr.linrec_last_error_message() or "1 GiB" in lr.linrec_last_error_message()


def test_interleaved_rows_of_h_that_do_not_overlap_are_refused_by_the_nesting_rule():
    """D=1, L=3 rows at time stride 2 and B=2 at batch stride 3: row starts {0, 2, 4} and {3, 5, 7}
    are disjoint, but the time rows interleave with the batch rows, which the nesting rule of
    linrec_scan_desc refuses; the nested form of the same rows (batch stride 6) is accepted."""
    assert not rows_overlap(2, 3, 1, 3, 2)
    for sb, ok in ((3, False), (6, True)):
        d = lr.linrec_scan_desc()
        d.B, d.L, d.D, d.dtype, d.reverse = 2, 3, 1, lr.LINREC_F32, 0
        for name in ("a", "b", "h"):
            setattr(d, name, lr.linrec_operand(BASE, sb, 2))
        plan = lr.linrec_plan()
        status = lr.library().linrec_scan_ex_plan(ctypes.byref(d), ctypes.byref(plan))
        assert (status == lr.LINREC_OK) == ok, (sb, lr.linrec_last_error_message())
