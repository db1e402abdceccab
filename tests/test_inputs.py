"""The seeded input generator: determinism, recipe and the named workloads.  CPU only."""
import numpy as np
import pytest

import linrec_inputs as li


def test_same_seed_same_bytes():
    a1, b1 = li.make_inputs(2, 50, 7, seed=9)
    a2, b2 = li.make_inputs(2, 50, 7, seed=9)
    assert a1.tobytes() == a2.tobytes() and b1.tobytes() == b2.tobytes()
    a3, _ = li.make_inputs(2, 50, 7, seed=10)
    assert a3.tobytes() != a1.tobytes()


def test_draw_order_and_dtype():
    a, b = li.make_inputs(3, 20, 5, seed=4)
    rng = np.random.default_rng(4)
    ra = rng.random((3, 20, 5), dtype=np.float32)
    rb = rng.standard_normal((3, 20, 5), dtype=np.float32)
    assert np.array_equal(a, ra) and np.array_equal(b, rb)
    assert a.dtype == np.float32 and b.dtype == np.float32
    assert a.flags.c_contiguous and b.flags.c_contiguous


def test_uniform_range_and_resets():
    a, _ = li.make_inputs(4, 2000, 64, seed=5, a_lo=0.999, a_hi=1.0, reset=0.01)
    nz = a[a != 0]
    assert nz.min() >= np.float32(0.999) and nz.max() <= np.float32(1.0)
    frac = float((a == 0).mean())
    assert 0.009 < frac < 0.011


def test_normal_a():
    a, _ = li.make_inputs(2, 3000, 32, seed=6, a_dist="normal")
    assert (a < 0).mean() > 0.45 and np.abs(a).max() > 3.0


@pytest.mark.parametrize("name", sorted(li.WORKLOADS))
def test_named_workloads(name):
    w = li.WORKLOADS[name]
    assert len(w.seeds) == 3 and w.elements == w.B * w.L * w.D
    # the recipe at a reduced length keeps the workload's distribution
    a, b = li.make_inputs(w.B, 8, w.D, w.seeds[0], w.a_dist, w.a_lo, w.a_hi, w.reset)
    assert a.shape == (w.B, 8, w.D)
    lo = 0.0 if w.reset else w.a_lo
    assert a.min() >= lo and a.max() <= w.a_hi


def test_headline_workload_shape():
    w = li.WORKLOADS[li.HEADLINE]
    assert (w.B, w.L, w.D) == (32, 4096, 256)
