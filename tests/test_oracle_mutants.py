"""Planted mistakes in the oracle must each fail at least one pin.

Every mutant is a copy of ``oracle/linrec_oracle.c`` with one plausible mistake
substituted into its arithmetic or indexing, compiled with the same flags into a
temporary library on the CPU; one more mutant is the reversed pair combine that
the POPCORNBENCH "FW-GLM-5-1 l1_p9" transcript's block-per-channel kernel applies
(the prefix's a multiplies the new b, instead of the new a multiplying the
prefix's b).  This shows the pins would notice a dropped term, a wrong sign, a
transposed operand, a wrong index or stride, fp32 accumulation or a reversed
combine anywhere in the oracle.
"""
from functools import partial

import numpy as np
import pytest

import oracle
from tests import oracle_pins

RECURRENCE = "ht[d] = (double)at[d] * hprev[d] + (double)bt[d];"

C_MUTANTS = {
    "dropped_b_term": (RECURRENCE, "ht[d] = (double)at[d] * hprev[d];"),
    "wrong_sign": (RECURRENCE, "ht[d] = (double)at[d] * hprev[d] - (double)bt[d];"),
    "a_b_transposed": (RECURRENCE, "ht[d] = (double)bt[d] * hprev[d] + (double)at[d];"),
    "fp32_accumulation": (RECURRENCE,
                          "ht[d] = (double)(float)((float)at[d] * (float)hprev[d] + (float)bt[d]);"),
    "a_index_off_by_one": ("const float *at = ab + t * D;", "const float *at = ab + (t - 1) * D;"),
    "stale_state_two_back": ("const double *hprev = hb + (t - 1) * D;",
                             "const double *hprev = hb + (t > 1 ? t - 2 : 0) * D;"),
    "initial_state_one": ("hb[d] = (double)bb[d];", "hb[d] = (double)ab[d] + (double)bb[d];"),
    "carry_skips_a0": ("hb[d] = (double)ab[d] * h_init[bi * D + d] + (double)bb[d];",
                       "hb[d] = h_init[bi * D + d] + (double)bb[d];"),
    "wrong_batch_stride": ("const float *ab = a + bi * L * D;", "const float *ab = a + bi * D;"),
}


REV_RECURRENCE = "rht[d] = (double)rat[d] * hnext[d] + (double)rbt[d];"

# mistakes in the reverse-time loop; caught by the reverse pins
REV_MUTANTS = {
    "rev_dropped_b_term": (REV_RECURRENCE, "rht[d] = (double)rat[d] * hnext[d];"),
    "rev_a_b_transposed": (REV_RECURRENCE, "rht[d] = (double)rbt[d] * hnext[d] + (double)rat[d];"),
    "rev_a_index_shift": ("const float *rat = rab + t * D;", "const float *rat = rab + (t + 1) * D;"),
    "rev_stale_state_two_ahead": ("const double *hnext = rhb + (t + 1) * D;",
                                  "const double *hnext = rhb + (t + 2 < L ? t + 2 : t + 1) * D;"),
    "rev_final_state_uses_a": ("rhb[last + d] = (double)rbb[last + d];",
                               "rhb[last + d] = (double)rab[last + d] + (double)rbb[last + d];"),
    "rev_carry_skips_a": ("rhb[last + d] = (double)rab[last + d] * h_init[bi * D + d] + (double)rbb[last + d];",
                          "rhb[last + d] = h_init[bi * D + d] + (double)rbb[last + d];"),
    "rev_wrong_batch_stride": ("const float *rbb = b_in + bi * L * D;", "const float *rbb = b_in + bi * D;"),
    "rev_fp32_accumulation": (REV_RECURRENCE,
                              "rht[d] = (double)(float)((float)rat[d] * (float)hnext[d] + (float)rbt[d]);"),
}


def _first_failing_pin(fn):
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(fn)
        except AssertionError:
            return pin.__name__
    return None


def _first_failing_rev_pin(f_rev, f_fwd):
    for pin in oracle_pins.REV_PINS:
        try:
            pin(f_rev, f_fwd)
        except AssertionError:
            return pin.__name__
    return None


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_c_mutant_is_caught(name, tmp_path):
    old, new = C_MUTANTS[name]
    src = oracle.SOURCE.read_text()
    assert src.count(old) == 1, f"mutation target not found exactly once: {old!r}"
    mutant_c = tmp_path / f"{name}.c"
    mutant_c.write_text(src.replace(old, new))
    lib = oracle.load_library(oracle.build(mutant_c, tmp_path / f"lib{name}.so"))
    caught = _first_failing_pin(partial(oracle.call_library, lib))
    assert caught is not None, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(REV_MUTANTS))
def test_reverse_c_mutant_is_caught(name, tmp_path):
    old, new = REV_MUTANTS[name]
    src = oracle.SOURCE.read_text()
    assert src.count(old) == 1, f"mutation target not found exactly once: {old!r}"
    mutant_c = tmp_path / f"{name}.c"
    mutant_c.write_text(src.replace(old, new))
    lib = oracle.load_library(oracle.build(mutant_c, tmp_path / f"lib{name}.so"))
    f_rev = partial(oracle.call_library, lib, reverse=True)
    caught = _first_failing_rev_pin(f_rev, oracle.linrec_oracle_f64)
    assert caught is not None, f"mutant {name} passed every reverse pin"


def _reversed_combine_oracle(a, b, h_init=None):
    """The oracle with the reversed combine: running pair (A, Bv) <- (A*a_t, A*b_t + Bv)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    h = np.empty(a.shape)
    if a.size == 0:
        return h
    A = a[:, 0, :].copy()
    Bv = b[:, 0, :].copy()
    if h_init is not None:
        Bv = Bv + A * np.asarray(h_init, np.float64)
    h[:, 0, :] = Bv
    for t in range(1, a.shape[1]):
        Bv = A * b[:, t, :] + Bv
        A = A * a[:, t, :]
        h[:, t, :] = Bv
    return h


def test_reversed_combine_is_caught():
    assert _first_failing_pin(_reversed_combine_oracle) is not None


def test_unmodified_copy_passes(tmp_path):
    """Control: the same build route with no substitution passes every pin."""
    c = tmp_path / "copy.c"
    c.write_text(oracle.SOURCE.read_text())
    lib = oracle.load_library(oracle.build(c, tmp_path / "libcopy.so"))
    assert _first_failing_pin(partial(oracle.call_library, lib)) is None
    assert _first_failing_rev_pin(partial(oracle.call_library, lib, reverse=True), oracle.linrec_oracle_f64) is None
