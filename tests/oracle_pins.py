"""Pins for the float64 oracle.

Each ``pin_*`` function takes an oracle callable ``f(a, b, h_init=None) ->
float64 (B, L, D) array`` and raises ``AssertionError`` when the callable
disagrees with something the pages or mathematics fix independently of the
oracle's own code: closed forms, a library routine (``scipy.signal.lfilter``),
exact rational brute force over random bracketings of the pair combine, the
pages' symbolic worked values (``tests/golden/worked_values.txt``), and exact
invariants of the recurrence.  ``tests/test_oracle_pins.py`` runs them against
the real oracle; ``tests/test_oracle_mutants.py`` runs them against planted
mistakes (dropped term, wrong sign, transposed operands, wrong index or stride,
reversed combine, fp32 accumulation) and requires every mistake to be caught.

The recurrence (POPCORNBENCH "Kimi-K2.6 l1_p9", problem statement):
h_0 = b_0, h_t = a_t * h_{t-1} + b_t over (B, L, D) with D contiguous.
The pair combine (same transcript, first reasoning block, operator
derivation): applying (a1, b1) then (a2, b2) equals (a2*a1, a2*b1 + b2),
identity (1, 0), and h_t is the second component of the inclusive scan when
the state before t = 0 is zero.
"""
from __future__ import annotations

import ast
import math
import random
from fractions import Fraction
from pathlib import Path

import numpy as np
from scipy.signal import lfilter

GOLDEN = Path(__file__).resolve().parent / "golden"


def _rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _close(h, ref, tol, what):
    h = np.asarray(h, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert h.shape == ref.shape, f"{what}: shape {h.shape} != {ref.shape}"
    ratio = np.abs(h - ref) / (1.0 + np.abs(ref))
    worst = float(np.max(ratio)) if ratio.size else 0.0
    assert np.all(np.isfinite(h)) and worst <= tol, f"{what}: max |h-ref|/(1+|ref|) = {worst:.3e} > {tol:.1e}"


def _bitwise(h, ref, what):
    h = np.asarray(h, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert h.shape == ref.shape, f"{what}: shape {h.shape} != {ref.shape}"
    # array_equal treats +0.0 and -0.0 as equal, which is the sign-of-zero allowance.
    bad = ~((h == ref) | (np.isnan(h) & np.isnan(ref)))
    assert not bad.any(), f"{what}: {int(bad.sum())} elements differ, first at {np.argwhere(bad)[0].tolist()}"


# --------------------------------------------------------------------------- closed forms

def pin_zero_a(f):
    """a == 0 everywhere: every step forgets the past, so h == b exactly."""
    rng = _rng(101)
    b = _normal(rng, (3, 37, 5))
    a = np.zeros_like(b)
    _bitwise(f(a, b), b, "a=0 -> h=b")


def pin_unit_a_prefix_sum(f):
    """a == 1 everywhere: h_t is the prefix sum of b, compared with math.fsum (correctly rounded)."""
    rng = _rng(102)
    B, L, D = 2, 300, 3
    b = _normal(rng, (B, L, D))
    a = np.ones_like(b)
    ref = np.empty((B, L, D))
    for bi in range(B):
        for d in range(D):
            col = b[bi, :, d].astype(np.float64).tolist()
            for t in range(L):
                ref[bi, t, d] = math.fsum(col[: t + 1])
    _close(f(a, b), ref, 1e-12, "a=1 -> prefix sum")


def pin_constant_a_lfilter(f):
    """a == c everywhere: h is the IIR filter y[n] = b[n] + c*y[n-1] with zero initial state,
    evaluated by scipy.signal.lfilter([1], [1, -c], b)."""
    rng = _rng(103)
    for c, L in ((0.5, 200), (-0.75, 200), (0.999, 400), (1.01, 150), (-1.3, 60)):
        cf = np.float32(c)
        b = _normal(rng, (2, L, 3))
        a = np.full_like(b, cf)
        ref = lfilter([1.0], [1.0, -float(cf)], b.astype(np.float64), axis=1)
        _close(f(a, b), ref, 1e-12, f"a={c} -> lfilter")


def pin_closed_form(f):
    """Time-varying a: h_t = sum_{s<=t} b_s * prod_{r=s+1..t} a_r, evaluated exactly in rationals."""
    rng = _rng(104)
    B, L, D = 2, 24, 3
    a = (rng.random((B, L, D), dtype=np.float32) * np.float32(3.0) - np.float32(1.5)).astype(np.float32)
    b = _normal(rng, (B, L, D))
    ref = np.empty((B, L, D))
    for bi in range(B):
        for d in range(D):
            af = [Fraction(float(x)) for x in a[bi, :, d]]
            bf = [Fraction(float(x)) for x in b[bi, :, d]]
            for t in range(L):
                total = Fraction(0)
                for s in range(t + 1):
                    prod = Fraction(1)
                    for r in range(s + 1, t + 1):
                        prod *= af[r]
                    total += bf[s] * prod
                ref[bi, t, d] = float(total)
    _close(f(a, b), ref, 1e-12, "closed form sum_s b_s prod a_r")


# --------------------------------------------------------------------------- exact brute force

def _compose(earlier, later):
    """Affine pair for 'apply earlier, then later'."""
    (a1, b1), (a2, b2) = earlier, later
    return (a2 * a1, a2 * b1 + b2)


def _fold_random(pairs, lo, hi, rnd):
    """Compose pairs[lo:hi] in order, splitting the range at random points (a random bracketing)."""
    if hi - lo == 1:
        return pairs[lo]
    mid = rnd.randint(lo + 1, hi - 1)
    return _compose(_fold_random(pairs, lo, mid, rnd), _fold_random(pairs, mid, hi, rnd))


def exact_sequential(a_col, b_col):
    """Exact rational h for one channel, stepping the definition."""
    h = []
    state = Fraction(0)
    for t, (x, y) in enumerate(zip(a_col, b_col)):
        state = Fraction(float(y)) if t == 0 else Fraction(float(x)) * state + Fraction(float(y))
        h.append(state)
    return h


def pin_bruteforce_bracketings(f):
    """On tiny inputs every fp32 value is an exact dyadic rational.  The sequential definition and a
    fold of the affine pairs under the combine, with random bracketings, must agree exactly; the
    oracle must match both within float64 rounding; the reversed combine must not."""
    rng = _rng(105)
    rnd = random.Random(105)
    B, L, D = 2, 12, 3
    a = (rng.random((B, L, D), dtype=np.float32) * np.float32(4.0) - np.float32(2.0)).astype(np.float32)
    b = _normal(rng, (B, L, D))
    ref = np.empty((B, L, D))
    reversed_differs = False
    for bi in range(B):
        for d in range(D):
            seq = exact_sequential(a[bi, :, d], b[bi, :, d])
            # a_0 multiplies the zero state, so the first pair's a can be anything; use 0.
            pairs = [(Fraction(0) if t == 0 else Fraction(float(a[bi, t, d])), Fraction(float(b[bi, t, d])))
                     for t in range(L)]
            for t in range(L):
                for _ in range(3):
                    A, Bv = _fold_random(pairs, 0, t + 1, rnd)
                    assert Bv == seq[t], "random bracketing changed the exact result"
                # the same fold with the operands of the combine swapped (the reversed operator)
                rev = pairs[0]
                for p in pairs[1:t + 1]:
                    rev = (rev[0] * p[0], rev[0] * p[1] + rev[1])
                reversed_differs |= rev[1] != seq[t]
                ref[bi, t, d] = float(seq[t])
    assert reversed_differs, "inputs too degenerate to tell the combine from its reverse"
    _close(f(a, b), ref, 1e-13, "exact rational brute force")


# --------------------------------------------------------------------------- the pages' worked values

def _eval_expr(expr: str, env: dict):
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.BinOp) and isinstance(node.op, (ast.Add, ast.Mult)):
            lhs, rhs = ev(node.left), ev(node.right)
            return lhs + rhs if isinstance(node.op, ast.Add) else lhs * rhs
        if isinstance(node, ast.Name):
            return env[node.id]
        raise ValueError(f"unsupported expression element {ast.dump(node)}")
    return ev(ast.parse(expr, mode="eval"))


def load_worked_values():
    rows = []
    for line in (GOLDEN / "worked_values.txt").read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, expr = (s.strip() for s in line.split("=", 1))
        rows.append((int(name[1:]), expr))
    return rows


def pin_worked_values(f):
    """The pages' symbolic h_0, h_1, h_2, evaluated exactly on random inputs."""
    rows = load_worked_values()
    assert [t for t, _ in rows] == [0, 1, 2]
    rng = _rng(106)
    D = 4
    a = (rng.random((1, 3, D), dtype=np.float32) * np.float32(4.0) - np.float32(2.0)).astype(np.float32)
    a[0, 0, :] = np.float32(7.5)   # a_0 appears in no expression; a large value exposes any use of it
    b = _normal(rng, (1, 3, D))
    ref = np.empty((1, 3, D))
    for d in range(D):
        env = {}
        for t in range(3):
            env[f"a{t}"] = Fraction(float(a[0, t, d]))
            env[f"b{t}"] = Fraction(float(b[0, t, d]))
        for t, expr in rows:
            ref[0, t, d] = float(_eval_expr(expr, env))
    _close(f(a, b), ref, 1e-15, "worked values h0, h1, h2")


# --------------------------------------------------------------------------- invariants

def pin_length_one(f):
    """L == 1: h = b, whatever a_0 is (it multiplies the zero state)."""
    rng = _rng(107)
    b = _normal(rng, (4, 1, 6))
    a = np.full_like(b, np.float32(np.inf))
    a[0, 0, :3] = np.float32(np.nan)
    a[1] = np.float32(-3.0)
    _bitwise(f(a, b), b, "L=1 -> h=b")


def pin_empty(f):
    """Any zero extent gives an empty result of the same shape."""
    for shape in ((0, 5, 3), (2, 0, 3), (2, 5, 0)):
        a = np.zeros(shape, np.float32)
        h = f(a, a.copy())
        assert h.shape == shape, f"empty {shape}: got {h.shape}"


def pin_impulse_layout(f):
    """A single unit impulse in b with a == 1/2 gives 2^-(t-t0) in that one channel after t0 and
    exact zeros everywhere else: pins the (B, L, D) strides and channel independence."""
    B, L, D = 3, 20, 5
    for (bs, ts, ds) in ((0, 0, 0), (2, 7, 3), (1, 19, 4), (1, 3, 0)):
        a = np.full((B, L, D), np.float32(0.5))
        b = np.zeros((B, L, D), np.float32)
        b[bs, ts, ds] = 1.0
        ref = np.zeros((B, L, D))
        for t in range(ts, L):
            ref[bs, t, ds] = 0.5 ** (t - ts)
        _bitwise(f(a, b), ref, f"impulse at {(bs, ts, ds)}")


def pin_reset(f):
    """Where a_t == 0, h_t == b_t exactly, and h from t on depends only on inputs from t on."""
    rng = _rng(108)
    B, L, D = 2, 100, 6
    a = rng.random((B, L, D), dtype=np.float32)
    b = _normal(rng, (B, L, D))
    mask = rng.random((B, L, D), dtype=np.float32) < np.float32(0.05)
    mask[1, 40, 2] = True
    a[mask] = 0.0
    h = f(a, b)
    _bitwise(h[mask], b[mask].astype(np.float64), "h==b at resets")
    # perturb everything strictly before the reset at (1, 40, 2) in that channel
    a2, b2 = a.copy(), b.copy()
    a2[1, :40, 2] = rng.random(40, dtype=np.float32) + np.float32(0.5)
    b2[1, :40, 2] = _normal(rng, (40,))
    h2 = f(a2, b2)
    _bitwise(h2[1, 40:, 2], h[1, 40:, 2], "reset cuts dependence on the past")


def pin_split_carry(f):
    """Scanning [k, L) from the state h_{k-1} reproduces the tail of the full scan exactly; a zero
    initial state reproduces the scan without one."""
    rng = _rng(109)
    B, L, D = 2, 64, 5
    a = (rng.random((B, L, D), dtype=np.float32) * np.float32(2.0) - np.float32(1.0)).astype(np.float32)
    b = _normal(rng, (B, L, D))
    h = f(a, b)
    for k in (1, 17, 63):
        tail = f(np.ascontiguousarray(a[:, k:]), np.ascontiguousarray(b[:, k:]), h_init=h[:, k - 1])
        _bitwise(tail, h[:, k:], f"split at {k}")
    _bitwise(f(a, b, h_init=np.zeros((B, D))), h, "zero initial state")
    # with a non-zero initial state the first step uses a_0: h_0 = a_0*h_init + b_0
    hi = _normal(rng, (B, D)).astype(np.float64)
    h0 = f(a, b, h_init=hi)[:, 0, :]
    ref0 = np.array([[float(Fraction(float(a[i, 0, d])) * Fraction(float(hi[i, d])) + Fraction(float(b[i, 0, d])))
                      for d in range(D)] for i in range(B)])
    _close(h0, ref0, 1e-15, "first step from a given state")


def pin_linearity(f):
    """h is linear in b for fixed a: exact under power-of-two scaling, additive within rounding.
    b1 and b2 are multiples of 1/64 below 2^7, so b1 + b2 is exact in fp32."""
    rng = _rng(110)
    B, L, D = 2, 80, 4
    a = (rng.random((B, L, D), dtype=np.float32) * np.float32(2.2) - np.float32(1.1)).astype(np.float32)
    b1 = (np.round(_normal(rng, (B, L, D)) * 64.0) / 64.0).astype(np.float32)
    b2 = (np.round(_normal(rng, (B, L, D)) * 64.0) / 64.0).astype(np.float32)
    bs = (b1 + b2).astype(np.float32)
    assert np.array_equal(bs.astype(np.float64), b1.astype(np.float64) + b2.astype(np.float64))
    h1, h2 = f(a, b1), f(a, b2)
    _bitwise(f(a, (b1 * np.float32(4.0)).astype(np.float32)), 4.0 * h1, "h(4b) = 4h(b)")
    err = np.abs(f(a, bs) - h1 - h2) / (1.0 + np.abs(h1) + np.abs(h2))
    assert float(err.max()) <= 1e-12, f"additivity in b: {float(err.max()):.3e}"


def pin_causality(f):
    """Changing inputs after time t0 leaves h up to t0 bitwise unchanged."""
    rng = _rng(111)
    B, L, D = 2, 50, 3
    a = rng.random((B, L, D), dtype=np.float32)
    b = _normal(rng, (B, L, D))
    h = f(a, b)
    t0 = 21
    a2, b2 = a.copy(), b.copy()
    a2[:, t0 + 1:] = rng.random((B, L - t0 - 1, D), dtype=np.float32) * np.float32(3.0)
    b2[:, t0 + 1:] = _normal(rng, (B, L - t0 - 1, D))
    _bitwise(f(a2, b2)[:, : t0 + 1], h[:, : t0 + 1], "causality")


def pin_equivariance(f):
    """Permuting batch rows and channels permutes the output the same way, bitwise."""
    rng = _rng(112)
    B, L, D = 3, 40, 7
    a = rng.random((B, L, D), dtype=np.float32)
    b = _normal(rng, (B, L, D))
    h = f(a, b)
    pb = rng.permutation(B)
    pd = rng.permutation(D)
    ap = np.ascontiguousarray(a[pb][:, :, pd])
    bp = np.ascontiguousarray(b[pb][:, :, pd])
    _bitwise(f(ap, bp), h[pb][:, :, pd], "permutation equivariance")


# --------------------------------------------------------------------------- reverse-time form
#
# The reverse-time recurrence h_t = a_t * h_{t+1} + b_t (t = L-1 .. 0, zero state after the last
# step) is not on the pages; it is the time reversal of their definition and the recurrence of the
# scan's gradient.  Each ``pin_rev_*`` takes the reverse oracle ``f_rev(a, b, h_init=None)`` and the
# forward oracle ``f_fwd`` (already pinned above) and checks f_rev against mathematics that does not
# go through its own loop.


def exact_reverse_closed_form(a_col, b_col):
    """Exact rational h for one channel: h_t = sum_{s>=t} b_s * prod_{r=t..s-1} a_r."""
    af = [Fraction(float(x)) for x in a_col]
    bf = [Fraction(float(x)) for x in b_col]
    L = len(bf)
    out = []
    for t in range(L):
        total, prod = Fraction(0), Fraction(1)
        for s in range(t, L):
            total += bf[s] * prod
            prod *= af[s]
        out.append(total)
    return out


def pin_rev_closed_form(f_rev, f_fwd):
    """Time-varying a, evaluated exactly in rationals; a_{L-1} multiplies the zero state only."""
    rng = _rng(201)
    B, L, D = 2, 20, 3
    a = (rng.random((B, L, D), dtype=np.float32) * np.float32(3.0) - np.float32(1.5)).astype(np.float32)
    b = _normal(rng, (B, L, D))
    ref = np.empty((B, L, D))
    for bi in range(B):
        for d in range(D):
            ref[bi, :, d] = [float(x) for x in exact_reverse_closed_form(a[bi, :, d], b[bi, :, d])]
    _close(f_rev(a, b), ref, 1e-12, "reverse closed form")
    a[:, -1, :] = np.float32(np.inf)
    _close(f_rev(a, b), ref, 1e-12, "reverse: a_{L-1} never used from a zero state")


def pin_rev_adjoint(f_rev, f_fwd):
    """The reverse recurrence over g with a shifted one step is the adjoint of the forward scan in b:
    per channel, sum_t g_t * fwd(a, b)_t == sum_t rev(a', g)_t * b_t with a'_t = a_{t+1}.  This is
    what makes it the gradient dLoss/db for g = dLoss/dh."""
    rng = _rng(202)
    B, L, D = 3, 300, 5
    a = (rng.random((B, L, D), dtype=np.float32) * np.float32(2.2) - np.float32(1.1)).astype(np.float32)
    b = _normal(rng, (B, L, D))
    g = _normal(rng, (B, L, D))
    a_next = np.zeros_like(a)
    a_next[:, :-1, :] = a[:, 1:, :]
    h = f_fwd(a, b)
    y = f_rev(a_next, g)
    lhs = np.sum(g.astype(np.float64) * h, axis=1)
    rhs = np.sum(y * b.astype(np.float64), axis=1)
    scale = np.sum(np.abs(g.astype(np.float64) * h), axis=1) + np.sum(np.abs(y * b.astype(np.float64)), axis=1)
    rel = np.abs(lhs - rhs) / scale
    assert float(rel.max()) <= 1e-12, f"adjoint identity: {float(rel.max()):.3e}"


def pin_rev_zero_a(f_rev, f_fwd):
    rng = _rng(203)
    b = _normal(rng, (3, 29, 4))
    _bitwise(f_rev(np.zeros_like(b), b), b, "reverse a=0 -> h=b")


def pin_rev_unit_a_suffix_sum(f_rev, f_fwd):
    """a == 1: h_t is the suffix sum of b from t on, compared with math.fsum."""
    rng = _rng(204)
    B, L, D = 2, 250, 3
    b = _normal(rng, (B, L, D))
    ref = np.empty((B, L, D))
    for bi in range(B):
        for d in range(D):
            col = b[bi, :, d].astype(np.float64).tolist()
            for t in range(L):
                ref[bi, t, d] = math.fsum(col[t:])
    _close(f_rev(np.ones_like(b), b), ref, 1e-12, "reverse a=1 -> suffix sum")


def pin_rev_split_carry(f_rev, f_fwd):
    """Scanning [0, k) backward from the state h_k reproduces the head of the full reverse scan
    exactly; a given final state enters as h_{L-1} = a_{L-1} * h_init + b_{L-1}."""
    rng = _rng(205)
    B, L, D = 2, 60, 5
    a = (rng.random((B, L, D), dtype=np.float32) * np.float32(2.0) - np.float32(1.0)).astype(np.float32)
    b = _normal(rng, (B, L, D))
    h = f_rev(a, b)
    for k in (1, 23, 59):
        head = f_rev(np.ascontiguousarray(a[:, :k]), np.ascontiguousarray(b[:, :k]), h_init=h[:, k])
        _bitwise(head, h[:, :k], f"reverse split at {k}")
    hi = _normal(rng, (B, D)).astype(np.float64)
    last = f_rev(a, b, h_init=hi)[:, -1, :]
    ref = np.array([[float(Fraction(float(a[i, -1, d])) * Fraction(float(hi[i, d])) + Fraction(float(b[i, -1, d])))
                     for d in range(D)] for i in range(B)])
    _close(last, ref, 1e-15, "reverse: last step from a given state")


def pin_rev_anticausal(f_rev, f_fwd):
    """Changing inputs before t0 leaves h from t0 on bitwise unchanged."""
    rng = _rng(206)
    B, L, D = 2, 50, 3
    a = rng.random((B, L, D), dtype=np.float32)
    b = _normal(rng, (B, L, D))
    h = f_rev(a, b)
    t0 = 19
    a2, b2 = a.copy(), b.copy()
    a2[:, :t0] = rng.random((B, t0, D), dtype=np.float32) * np.float32(3.0)
    b2[:, :t0] = _normal(rng, (B, t0, D))
    _bitwise(f_rev(a2, b2)[:, t0:], h[:, t0:], "anti-causality")


def pin_rev_length_one_and_empty(f_rev, f_fwd):
    rng = _rng(207)
    b = _normal(rng, (3, 1, 4))
    _bitwise(f_rev(np.full_like(b, np.float32(np.inf)), b), b, "reverse L=1 -> h=b")
    for shape in ((0, 5, 3), (2, 0, 3), (2, 5, 0)):
        z = np.zeros(shape, np.float32)
        assert f_rev(z, z.copy()).shape == shape


REV_PINS = [
    pin_rev_closed_form,
    pin_rev_adjoint,
    pin_rev_zero_a,
    pin_rev_unit_a_suffix_sum,
    pin_rev_split_carry,
    pin_rev_anticausal,
    pin_rev_length_one_and_empty,
]


ALL_PINS = [
    pin_zero_a,
    pin_unit_a_prefix_sum,
    pin_constant_a_lfilter,
    pin_closed_form,
    pin_bruteforce_bracketings,
    pin_worked_values,
    pin_length_one,
    pin_empty,
    pin_impulse_layout,
    pin_reset,
    pin_split_carry,
    pin_linearity,
    pin_causality,
    pin_equivariance,
]
