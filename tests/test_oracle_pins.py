"""The float64 oracle against its pins (closed forms, library routines, exact brute force,
the pages' worked values, invariants).  CPU only."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.linrec_oracle_f64)


@pytest.mark.parametrize("pin", oracle_pins.REV_PINS, ids=lambda p: p.__name__)
def test_reverse_oracle_pin(pin):
    pin(oracle.linrec_oracle_rev_f64, oracle.linrec_oracle_f64)


def test_thread_count_does_not_change_bits():
    rng = np.random.default_rng(7)
    a = rng.random((3, 200, 150), dtype=np.float32)
    b = rng.standard_normal((3, 200, 150), dtype=np.float32)
    for fn in (oracle.linrec_oracle_f64, oracle.linrec_oracle_rev_f64):
        assert np.array_equal(fn(a, b, threads=1), fn(a, b, threads=5))


def test_rejects_mismatched_shapes():
    a = np.zeros((2, 3, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.linrec_oracle_f64(a, np.zeros((2, 3, 5), np.float32))
    with pytest.raises(ValueError):
        oracle.linrec_oracle_f64(a, a, h_init=np.zeros((2, 5)))
