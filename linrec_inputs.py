"""Seeded synthetic inputs for the linear-recurrence scan.

This module is shared by the tests, the benchmark and the smoke check, and it
feeds both the HIP path and the float64 oracle with identical bytes.  It holds
none of the recurrence's arithmetic: it only draws random numbers.

Recipe (fixed, so that every consumer sees the same bytes for a given seed):

* generator ``numpy.random.default_rng(seed)`` (PCG64);
* draw order: ``a`` first, then ``b``, then the reset mask (if any);
* ``a`` ~ U[lo, hi) computed in fp32 as ``lo + (hi - lo) * U[0,1)`` (may round
  to ``hi``), or N(0,1) for the "normal" case;
* ``b`` ~ N(0,1), ``standard_normal`` in fp32;
* reset mask: an i.i.d. Bernoulli(p) draw per element (b, t, d), taken as
  ``U[0,1) < p`` in fp32, sets ``a`` to 0 at those positions;
* arrays are fp32, C-contiguous, shape (B, L, D) with D fastest.

The five named workloads are the shapes and distributions of the
linear-recurrence scan problem studied on the POPCORNBENCH "l1_p9" transcripts
(B=32, L=4096, D=256, inputs drawn with ``randn``) together with four more
shapes that stress the other regimes of the method: a tiny case, a long
sequence with few channels, many channels with a short sequence, and a
near-unit decay with resets.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    L: int
    D: int
    a_dist: str = "uniform"      # "uniform" or "normal"
    a_lo: float = 0.0
    a_hi: float = 1.0
    reset: float = 0.0           # probability that a position is a reset (a = 0)
    seeds: tuple = (0,)

    @property
    def shape(self):
        return (self.B, self.L, self.D)

    @property
    def elements(self) -> int:
        return self.B * self.L * self.D

    def describe(self, storage: str = "fp32") -> str:
        """Shape, storage type and distributions; ``storage`` names the type a, b and h are held
        in (the values are drawn in fp32 and, for 16-bit storage, rounded to it)."""
        if self.a_dist == "normal":
            a = "a~N(0,1)"
        else:
            a = f"a~U({self.a_lo:g},{self.a_hi:g})"
        extra = f", {self.reset:.0%} resets a=0" if self.reset else ""
        return f"B={self.B} L={self.L} D={self.D} {storage}, {a}, b~N(0,1){extra}"


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 8, seeds=(1, 11, 21)),
    "pages_shape": Workload("pages_shape", 32, 4096, 256, seeds=(2, 12, 22)),
    "long_sequence": Workload("long_sequence", 2, 262144, 64, a_lo=0.9, a_hi=1.0, seeds=(3, 13, 23)),
    "wide_channels": Workload("wide_channels", 16, 512, 8192, seeds=(4, 14, 24)),
    "near_unit_resets": Workload("near_unit_resets", 8, 16384, 1024, a_lo=0.999, a_hi=1.0,
                                 reset=0.01, seeds=(5, 15, 25)),
}

# The workload the headline throughput is quoted on.
HEADLINE = "pages_shape"


def make_inputs(B: int, L: int, D: int, seed: int, a_dist: str = "uniform",
                a_lo: float = 0.0, a_hi: float = 1.0, reset: float = 0.0):
    """Return (a, b) fp32 arrays of shape (B, L, D) drawn by the recipe above."""
    rng = np.random.default_rng(seed)
    shape = (B, L, D)
    if a_dist == "uniform":
        a = rng.random(shape, dtype=np.float32)
        if (a_lo, a_hi) != (0.0, 1.0):
            a *= np.float32(a_hi - a_lo)
            a += np.float32(a_lo)
    elif a_dist == "normal":
        a = rng.standard_normal(shape, dtype=np.float32)
    else:
        raise ValueError(f"unknown a distribution {a_dist!r}")
    b = rng.standard_normal(shape, dtype=np.float32)
    if reset > 0.0:
        mask = rng.random(shape, dtype=np.float32) < np.float32(reset)
        a[mask] = 0.0
        del mask
    return a, b


def workload_inputs(name: str, seed: int | None = None):
    """(a, b) for a named workload; ``seed`` defaults to the workload's first seed."""
    w = WORKLOADS[name]
    s = w.seeds[0] if seed is None else seed
    return make_inputs(w.B, w.L, w.D, s, w.a_dist, w.a_lo, w.a_hi, w.reset)
