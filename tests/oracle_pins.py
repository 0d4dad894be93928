"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when that oracle is wrong.  ``test_oracle_pins.py`` runs them against the real
oracle; ``test_oracle_mutants.py`` runs them against copies of ``oracle.c``
with planted mistakes and requires every mistake to be caught.

What the pins rest on (none of them re-types the oracle's own loop):

* closed forms -- the harmonic number H_n for the README's synthetic input
  x[i] = 1/(i+1); a constant c summed n times is n*c; index-encoded data
  x[o, r, i] = o*B^2 + r*B + i sums over r to R*(o*B^2 + i) + B*R(R-1)/2;
* exactness -- integer-valued data is summed exactly by any order, so the
  oracle must equal the exact integer sum bit for bit;
* a correctly rounded library sum -- ``math.fsum`` (Shewchuk), with the
  sequential fp64 error bound (n-1) * 2^-53 * sum|x|;
* a library axis routine -- numpy's ``sum(axis=1)`` on integer data (exact);
* IEEE special cases -- NaN, +-Inf, signed zero, empty sums;
* for the other reductions: sum of squares closed forms (n(n+1)(2n+1)/6),
  exact integer sums of squares, numpy's max / min, IEEE 754-2019
  maximum / minimum special cases, order independence;
* for the softmax denominator: constant columns (every term exp(0) = 1),
  a shuffled geometric series (closed form (1 - q^R) / (1 - q)), shift
  invariance, scipy's and torch's log-sum-exp (independent library
  routines, special values included), numpy's max.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import workloads

EULER_GAMMA = 0.5772156649015329
U53 = 2.0 ** -53
U24 = 2.0 ** -24
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def harmonic_closed_form(n: int) -> float:
    """H_n = ln n + gamma + 1/(2n) - 1/(12 n^2) (next term: +1/(120 n^4))."""
    return math.log(n) + EULER_GAMMA + 1.0 / (2 * n) - 1.0 / (12.0 * n * n)


# --------------------------------------------------------------------------- 1D
def pin_harmonic(orc):
    """README synthetic input at n = 1e6 against the closed form of H_n.

    Each fp32 term carries a relative rounding error <= 2^-24, so the exact sum
    of the fp32 terms is within 2^-24 * H_n of H_n; the fp64 accumulation adds
    at most (n-1) * 2^-53 * H_n.  A single dropped term (>= 1e-6) breaks it.
    """
    n = 1_000_000
    x = workloads.harmonic(n)
    S, A = orc.sum_1d(x)
    H = harmonic_closed_form(n)
    assert abs(S - H) <= U24 * H + n * U53 * H, (S, H)
    assert S == A  # all terms positive
    # and tighter: against the correctly rounded sum of the same fp32 terms
    F = math.fsum(x.astype(np.float64).tolist())
    assert abs(S - F) <= (n - 1) * U53 * A, (S, F)


def pin_constants_1d(orc):
    """A constant c summed n times is exactly n*c (all partials exact in fp64)."""
    for c in (1.0, 0.5, -0.25, 3.0):
        for n in (0, 1, 2, 3, 4, 5, 7, 64, 1000, 12345):
            S, A = orc.sum_1d(np.full(n, c, dtype=np.float32))
            assert S == n * c and A == n * abs(c), (c, n, S, A)


def pin_integers_1d(orc):
    """Integer-valued data: the oracle equals the exact integer sum."""
    for seed, n in ((11, 1), (12, 17), (13, 4096), (14, 1_000_003)):
        x = workloads.small_ints(n, seed)
        exact = int(np.sum(x.astype(np.int64)))
        exact_abs = int(np.sum(np.abs(x.astype(np.int64))))
        S, A = orc.sum_1d(x)
        assert S == exact and A == exact_abs, (n, S, exact, A, exact_abs)


def pin_fsum_1d(orc):
    """Random data against math.fsum within the sequential fp64 error bound."""
    for seed, n, dist in ((21, 100_000, "normal"), (22, 1_000_000, "uniform"),
                          (23, 999_999, "normal")):
        lo, hi = (-1.0, 1.0) if dist == "uniform" else (0.0, 1.0)
        x = workloads.random(n, seed, dist, lo, hi)
        S, A = orc.sum_1d(x)
        F = math.fsum(x.astype(np.float64).tolist())
        Fa = math.fsum(np.abs(x.astype(np.float64)).tolist())
        assert abs(S - F) <= (n - 1) * U53 * A, (n, S, F)
        assert abs(A - Fa) <= (n - 1) * U53 * Fa, (n, A, Fa)


def pin_special_values_1d(orc):
    """IEEE propagation and signed zero; the empty sum is +0.0."""
    S, A = orc.sum_1d(np.zeros(0, dtype=np.float32))
    assert S == 0.0 and not math.copysign(1.0, S) < 0 and A == 0.0
    S, _ = orc.sum_1d(np.full(9, -0.0, dtype=np.float32))
    assert S == 0.0 and math.copysign(1.0, S) > 0, S
    S, _ = orc.sum_1d(np.array([-0.0], dtype=np.float32))
    assert math.copysign(1.0, S) > 0, S
    x = np.ones(100, dtype=np.float32)
    x[37] = np.nan
    S, _ = orc.sum_1d(x)
    assert math.isnan(S)
    x = np.ones(100, dtype=np.float32)
    x[5] = np.inf
    S, A = orc.sum_1d(x)
    assert S == math.inf and A == math.inf
    x[90] = -np.inf
    S, _ = orc.sum_1d(x)
    assert math.isnan(S)
    x = np.array([np.finfo(np.float32).max] * 4, dtype=np.float32)
    S, _ = orc.sum_1d(x)  # finite in fp64
    assert S == 4.0 * float(np.finfo(np.float32).max)
    x = np.array([1e-45, 1e-45, -1e-45], dtype=np.float32)  # denormals kept
    S, _ = orc.sum_1d(x)
    assert S == float(x[0]) + float(x[1]) + float(x[2]) and S != 0.0


# ------------------------------------------------------------------------- axis
AXIS_SHAPES = ((3, 5, 7), (2, 9, 1), (1, 4, 6), (4, 1, 3), (5, 3, 2), (1, 1, 1),
               (6, 33, 65), (2, 128, 4095 % 64 + 3))


def index_encoded(outer, R, inner, B=64):
    """x[o, r, i] = o*B^2 + r*B + i (exact in fp32 while < 2^24)."""
    o = np.arange(outer, dtype=np.int64)[:, None, None]
    r = np.arange(R, dtype=np.int64)[None, :, None]
    i = np.arange(inner, dtype=np.int64)[None, None, :]
    v = o * B * B + r * B + i
    assert v.size == 0 or v.max() < 2 ** 24
    return v.astype(np.float32).reshape(-1)


def pin_index_closed_form(orc):
    """Index-encoded data: sum over r is R*(o*B^2 + i) + B*R*(R-1)/2.

    A transposed operand, a wrong stride, a dropped or repeated row or a
    shifted column all change at least one output.
    """
    B = 64
    for outer, R, inner in AXIS_SHAPES:
        x = index_encoded(outer, R, inner, B)
        S, A = orc.sum_dim(x, outer, R, inner)
        o = np.arange(outer, dtype=np.float64)[:, None]
        i = np.arange(inner, dtype=np.float64)[None, :]
        want = R * (o * B * B + i) + B * R * (R - 1) / 2.0
        assert np.array_equal(S, want), (outer, R, inner)
        assert np.array_equal(A, want), (outer, R, inner)  # all terms >= 0
        # the per-output entry point on a sample of outputs
        oo, ii = np.meshgrid(np.arange(outer), np.arange(inner), indexing="ij")
        s1, a1 = orc.sum_dim_at(x, outer, R, inner, oo.reshape(-1), ii.reshape(-1))
        assert np.array_equal(s1, want.reshape(-1)), (outer, R, inner)
        assert np.array_equal(a1, want.reshape(-1)), (outer, R, inner)


def pin_constants_axis(orc):
    """A constant c summed over R rows is exactly R*c in every output."""
    for c in (1.0, 0.5, -0.25, 3.0):
        for outer, R, inner in AXIS_SHAPES + ((2, 0, 3), (0, 4, 4), (3, 2, 0)):
            x = np.full(outer * R * inner, c, dtype=np.float32)
            S, A = orc.sum_dim(x, outer, R, inner)
            assert S.shape == (outer, inner)
            assert np.all(S == R * c) and np.all(A == R * abs(c)), (c, outer, R, inner)


def pin_bruteforce_axis(orc):
    """Every shape in [0..4]^3 (and a few wider) with integer data against
    numpy's axis-1 sum in int64, which is exact."""
    shapes = [(a, b, c) for a in range(5) for b in range(5) for c in range(5)]
    shapes += [(3, 17, 63), (2, 64, 64), (1, 65, 129), (7, 3, 4095)]
    for k, (outer, R, inner) in enumerate(shapes):
        x = workloads.small_ints(outer * R * inner, 1000 + k)
        want = x.astype(np.int64).reshape(outer, R, inner).sum(axis=1)
        want_abs = np.abs(x.astype(np.int64)).reshape(outer, R, inner).sum(axis=1)
        S, A = orc.sum_dim(x, outer, R, inner, threads=2)
        assert np.array_equal(S, want.astype(np.float64)), (outer, R, inner)
        assert np.array_equal(A, want_abs.astype(np.float64)), (outer, R, inner)


def pin_fsum_axis(orc):
    """Sampled outputs of random data against math.fsum of the strided column,
    taken by numpy slicing (an indexing independent of the oracle's)."""
    rng = np.random.default_rng(5)
    for seed, (outer, R, inner) in ((31, (4, 1000, 37)), (32, (3, 4096, 5)),
                                    (33, (64, 300, 1))):
        x = workloads.random(outer * R * inner, seed, "normal")
        S, A = orc.sum_dim(x, outer, R, inner)
        x3 = x.reshape(outer, R, inner)
        for _ in range(20):
            o, i = int(rng.integers(outer)), int(rng.integers(inner))
            col = x3[o, :, i].astype(np.float64)
            F = math.fsum(col.tolist())
            assert abs(S[o, i] - F) <= (R - 1) * U53 * A[o, i], (o, i)
            assert abs(A[o, i] - math.fsum(np.abs(col).tolist())) <= R * U53 * A[o, i]


def pin_special_values_axis(orc):
    """NaN / Inf stay in their own output; signed zero gives +0.0."""
    outer, R, inner = 2, 5, 3
    x = np.ones(outer * R * inner, dtype=np.float32).reshape(outer, R, inner)
    x[1, 3, 2] = np.nan
    x[0, 0, 1] = np.inf
    S, _ = orc.sum_dim(x, outer, R, inner)
    assert math.isnan(S[1, 2]) and S[0, 1] == math.inf
    assert np.isfinite(np.delete(S.reshape(-1), [1, 5])).all()
    z = np.full(outer * R * inner, -0.0, dtype=np.float32)
    S, _ = orc.sum_dim(z, outer, R, inner)
    assert np.all(S == 0.0) and not np.any(np.signbit(S))


def pin_page_shape_facts(orc):
    """Shape arithmetic the problem-47 trace prints, checked against the
    workload definition (the oracle is exercised on the page's own shape
    family at a reduced R so the check stays small)."""
    with open(os.path.join(GOLDEN, "problem47_shape_facts.json")) as f:
        facts = json.load(f)
    w = workloads.WORKLOADS["cols_128x4096x4095"]
    assert list(w.shape) == facts["shape"]
    outer, R, inner = w.outer, w.R, w.inner
    assert R * inner == facts["slab_elements"]
    assert (R * inner) % 16 == facts["slab_elements_mod_16"]
    assert 4 * inner == facts["row_bytes"]
    assert (4 * inner) % 16 == facts["row_bytes_mod_16"]
    assert (4 * inner) % 128 == facts["row_bytes_over_128_line_offset"]
    assert (4 * inner) // 128 == facts["row_bytes_line_index"]
    assert w.out_numel == facts["outputs"]
    # the oracle on that outer/inner with 4 rows: output count and layout
    x = index_encoded(2, 4, inner, B=1)
    S, _ = orc.sum_dim(x, 2, 4, inner)
    assert S.size == 2 * inner


# ------------------------------------------------------ other reductions
def pin_sumsq_closed_form(orc):
    """x[i] = i + 1: sum of squares n(n+1)(2n+1)/6, exact in fp64 here; along
    an axis with x[o, r, i] = r + 1 every output is R(R+1)(2R+1)/6."""
    for n in (0, 1, 2, 7, 1000, 100_000):
        x = np.arange(1, n + 1, dtype=np.float32)
        S, A = orc.reduce_1d(x, "sumsq")
        want = n * (n + 1) * (2 * n + 1) // 6
        assert S == want and A == want, (n, S, want)
    for outer, R, inner in ((3, 5, 7), (2, 1000, 1), (1, 33, 65)):
        x = np.broadcast_to(np.arange(1, R + 1, dtype=np.float32)[None, :, None],
                            (outer, R, inner)).copy()
        S, _ = orc.reduce_dim(x, outer, R, inner, "sumsq")
        assert np.all(S == R * (R + 1) * (2 * R + 1) // 6), (outer, R, inner)


def pin_sumsq_exact_and_fsum(orc):
    """Integer data: the exact int64 sum of squares; random data: math.fsum of
    the (exact) fp64 squares within the sequential bound; axis brute force."""
    x = workloads.small_ints(1_000_003, 41)
    S, A = orc.reduce_1d(x, "sumsq")
    assert S == int(np.sum(x.astype(np.int64) ** 2)) and A == S
    y = workloads.random(200_000, 42, "normal")
    S, A = orc.reduce_1d(y, "sumsq")
    F = math.fsum((y.astype(np.float64) ** 2).tolist())
    assert abs(S - F) <= len(y) * U53 * A
    for k, (outer, R, inner) in enumerate(((3, 17, 63), (5, 4, 1), (2, 9, 4095))):
        z = workloads.small_ints(outer * R * inner, 43 + k)
        S, _ = orc.reduce_dim(z, outer, R, inner, "sumsq")
        want = (z.astype(np.int64).reshape(outer, R, inner) ** 2).sum(axis=1)
        assert np.array_equal(S, want.astype(np.float64)), (outer, R, inner)
        oo, ii = np.meshgrid(np.arange(outer), np.arange(inner), indexing="ij")
        s1, _ = orc.reduce_dim_at(z, outer, R, inner, "sumsq", oo.reshape(-1), ii.reshape(-1))
        assert np.array_equal(s1, want.reshape(-1).astype(np.float64))


def pin_max_min_library(orc):
    """Maximum and minimum of random data equal numpy's, along any axis, and
    do not depend on the order of the terms."""
    rng = np.random.default_rng(44)
    x = workloads.random(1_000_001, 45, "normal")
    for op, f in (("max", np.max), ("min", np.min)):
        S, A = orc.reduce_1d(x, op)
        assert S == float(f(x)) and A == abs(S)
        S2, _ = orc.reduce_1d(x[rng.permutation(x.size)], op)
        assert S2 == S
        assert orc.reduce_1d(-x, op)[0] == -orc.reduce_1d(x, "min" if op == "max" else "max")[0]
    for outer, R, inner in ((3, 5, 7), (4, 1000, 1), (2, 64, 4095), (1, 1, 3)):
        z = workloads.random(outer * R * inner, 46 + R, "uniform", -1.0, 1.0)
        z3 = z.reshape(outer, R, inner)
        for op, f in (("max", np.max), ("min", np.min)):
            S, _ = orc.reduce_dim(z, outer, R, inner, op)
            assert np.array_equal(S, f(z3, axis=1).astype(np.float64)), (op, outer, R, inner)
            oo, ii = np.meshgrid(np.arange(outer), np.arange(inner), indexing="ij")
            s1, _ = orc.reduce_dim_at(z, outer, R, inner, op, oo.reshape(-1), ii.reshape(-1))
            assert np.array_equal(s1, S.reshape(-1))
    # all-negative and all-positive data: the start values are -Inf / +Inf
    neg = -np.abs(x) - 1.0
    assert orc.reduce_1d(neg.astype(np.float32), "max")[0] == float(np.max(neg.astype(np.float32)))
    pos = np.abs(x) + 1.0
    assert orc.reduce_1d(pos.astype(np.float32), "min")[0] == float(np.min(pos.astype(np.float32)))


def pin_max_min_special(orc):
    """IEEE 754-2019 maximum / minimum: NaN propagates, -0 < +0 in either
    order, Inf is a value; the max of nothing is -Inf, the min +Inf."""
    f = lambda *v: np.array(v, dtype=np.float32)
    for v in (f(-0.0, 0.0), f(0.0, -0.0), f(-0.0, 0.0, -0.0)):
        S, _ = orc.reduce_1d(v, "max")
        assert S == 0.0 and not math.copysign(1.0, S) < 0, v
        S, _ = orc.reduce_1d(v, "min")
        assert S == 0.0 and math.copysign(1.0, S) < 0, v
    assert math.copysign(1.0, orc.reduce_1d(f(-0.0, -0.0), "max")[0]) < 0
    for op in ("max", "min", "sumsq"):
        for pos in (0, 3, 6):
            v = f(1, 2, 3, 4, 5, 6, 7)
            v[pos] = np.nan
            assert math.isnan(orc.reduce_1d(v, op)[0]), (op, pos)
    assert orc.reduce_1d(f(1, np.inf, 2), "max")[0] == math.inf
    assert orc.reduce_1d(f(1, -np.inf, 2), "min")[0] == -math.inf
    assert orc.reduce_1d(f(), "max")[0] == -math.inf
    assert orc.reduce_1d(f(), "min")[0] == math.inf
    assert orc.reduce_1d(f(), "sumsq")[0] == 0.0
    z = np.ones((2, 3, 4), np.float32)
    z[1, 2, 3] = np.nan
    S, _ = orc.reduce_dim(z, 2, 3, 4, "max")
    assert math.isnan(S[1, 3]) and np.isfinite(np.delete(S.reshape(-1), 7)).all()
    S, _ = orc.reduce_dim(np.zeros(0, np.float32), 2, 0, 3, "min")
    assert np.all(S == math.inf)


# ------------------------------------------------------ cumulative sums
def pin_cumsum_page_example(orc):
    """The problem-91 trace's worked row [a, b, c, d] -> [a+b+c+d, b+c+d,
    c+d, d] (tests/golden/problem91_reverse_cumsum.json), in every layout
    the row can take: alone, as one of several rows, as a column."""
    with open(os.path.join(GOLDEN, "problem91_reverse_cumsum.json")) as f:
        g = json.load(f)
    row = np.array(g["row"], np.float32)
    want = np.array(g["reverse_cumsum"])
    S, A = orc.cumsum_dim(row, 1, row.size, 1, True)
    assert np.array_equal(S.reshape(-1), want) and np.array_equal(A.reshape(-1), want)
    rows = np.stack([row, 2 * row, -row]).astype(np.float32)
    S, _ = orc.cumsum_dim(rows, 3, row.size, 1, True)
    assert np.array_equal(S.reshape(3, -1), np.stack([want, 2 * want, -want]))
    col = np.repeat(row[:, None], 5, axis=1).astype(np.float32)   # [R, inner]
    S, _ = orc.cumsum_dim(col, 1, row.size, 5, True)
    assert np.array_equal(S.reshape(row.size, 5), np.repeat(want[:, None], 5, axis=1))
    # forward: the running sum from the front
    S, _ = orc.cumsum_dim(row, 1, row.size, 1, False)
    assert np.array_equal(S.reshape(-1), np.cumsum(g["row"]))


def pin_cumsum_library(orc):
    """Integer data: the trace's own formula cumsum(x.flip(1), 1).flip(1)
    evaluated exactly by numpy in int64, and the forward cumsum; ones give
    R - r and r + 1."""
    for k, (outer, R, inner) in enumerate(((1, 1, 1), (3, 17, 1), (2, 64, 5), (4, 33, 4095),
                                           (5, 1000, 1), (2, 0, 3))):
        x = workloads.small_ints(outer * R * inner, 80 + k)
        x3 = x.astype(np.int64).reshape(outer, R, inner)
        rev = np.flip(np.cumsum(np.flip(x3, 1), 1), 1)
        fwd = np.cumsum(x3, 1)
        S, A = orc.cumsum_dim(x, outer, R, inner, True)
        assert np.array_equal(S, rev.astype(np.float64)), (outer, R, inner)
        absrev = np.flip(np.cumsum(np.flip(np.abs(x3), 1), 1), 1)
        assert np.array_equal(A, absrev.astype(np.float64))
        S, _ = orc.cumsum_dim(x, outer, R, inner, False)
        assert np.array_equal(S, fwd.astype(np.float64)), (outer, R, inner)
    ones = np.ones(3 * 50 * 2, np.float32)
    S, _ = orc.cumsum_dim(ones, 3, 50, 2, True)
    assert np.all(S == (50 - np.arange(50))[None, :, None])
    S, _ = orc.cumsum_dim(ones, 3, 50, 2, False)
    assert np.all(S == (1 + np.arange(50))[None, :, None])


def pin_cumsum_fsum(orc):
    """Random data: every output of a few rows against math.fsum of its terms
    within the sequential fp64 bound; the reverse sum's first element is the
    row sum."""
    R = 3000
    x = workloads.random(4 * R, 90, "normal").reshape(4, R)
    S, A = orc.cumsum_dim(x, 4, R, 1, True)
    S = S.reshape(4, R)
    A = A.reshape(4, R)
    for o in range(4):
        for j in (0, 1, 7, R // 2, R - 2, R - 1):
            F = math.fsum(x[o, j:].astype(np.float64).tolist())
            assert abs(S[o, j] - F) <= (R - j) * U53 * A[o, j], (o, j)
        Sr, _ = orc.sum_dim(x[o], 1, R, 1)
        assert abs(S[o, 0] - Sr[0, 0]) <= 2 * R * U53 * A[o, 0]


# ------------------------------------------------------ softmax denominator
def pin_softmax_constants(orc):
    """A constant column x_r = c has maximum c and every shifted term
    exp(c - c) = 1, so S = R exactly, for any c; no terms: (-Inf, 0)."""
    for c in (0.0, 1.0, -1000.0, 1000.0, 3.5, -0.125):
        for outer, R, inner in ((1, 1, 1), (2, 7, 3), (1, 1000, 1), (3, 5, 130)):
            x = np.full(outer * R * inner, c, np.float32)
            M, S = orc.softmax_denom_dim(x, outer, R, inner)
            assert np.all(M == c) and np.all(S == R), (c, outer, R, inner)
    M, S = orc.softmax_denom_dim(np.zeros(0, np.float32), 2, 0, 3)
    assert np.all(M == -math.inf) and np.all(S == 0.0)


def pin_softmax_geometric(orc):
    """Column (o, i) holds k - delta * p for p = 0 .. R-1 in a shuffled order
    (k an integer of either sign, delta exact in fp32): its maximum is k and
    S = sum_p q^p = (1 - q^R) / (1 - q) with q = exp(-delta), whatever k."""
    rng = np.random.default_rng(47)
    for outer, R, inner, delta in ((2, 20, 3, 0.5), (1, 300, 1, 0.25), (3, 9, 70, 1.0),
                                   (1, 1, 4, 0.5)):
        x = np.empty((outer, R, inner), np.float32)
        k = rng.integers(-60, 60, size=(outer, inner))
        for o in range(outer):
            for i in range(inner):
                x[o, :, i] = k[o, i] - delta * rng.permutation(R)
        M, S = orc.softmax_denom_dim(x, outer, R, inner)
        q = math.exp(-delta)
        want = (1.0 - q ** R) / (1.0 - q)
        assert np.array_equal(M, k.astype(np.float64)), (outer, R, inner)
        assert np.all(np.abs(S - want) <= 1e-13 * want), (outer, R, inner, S, want)
        oo, ii = np.meshgrid(np.arange(outer), np.arange(inner), indexing="ij")
        m1, s1 = orc.softmax_denom_dim_at(x, outer, R, inner, oo.reshape(-1), ii.reshape(-1))
        assert np.array_equal(m1, M.reshape(-1)) and np.array_equal(s1, S.reshape(-1))


def pin_softmax_library(orc):
    """Random data: the maximum equals numpy's; c + log S equals scipy's
    logsumexp along the same axis (an independent implementation); adding
    an integer to every term moves the maximum by it and leaves S alone."""
    from scipy.special import logsumexp
    for k, (outer, R, inner, scale) in enumerate(((3, 5, 7, 1.0), (4, 1000, 1, 10.0),
                                                  (2, 64, 4095, 3.0), (1, 1, 3, 1.0),
                                                  (5, 333, 2, 30.0))):
        x = workloads.random(outer * R * inner, 60 + k, "normal") * np.float32(scale)
        x3 = x.reshape(outer, R, inner)
        M, S = orc.softmax_denom_dim(x, outer, R, inner)
        assert np.array_equal(M, np.max(x3, axis=1).astype(np.float64)), (outer, R, inner)
        lse = logsumexp(x3.astype(np.float64), axis=1)
        assert np.all(np.abs(M + np.log(S) - lse) <= 1e-12 * (1 + np.abs(lse))), (outer, R, inner)
        assert np.all(S >= 1.0) and np.all(S <= R)
        for shift in (7, -40):
            M2, S2 = orc.softmax_denom_dim((x + np.float32(shift)).astype(np.float32), outer, R,
                                           inner)
            exact = (x + np.float32(shift)).astype(np.float64) == x.astype(np.float64) + shift
            if exact.all():
                assert np.array_equal(M2, M + shift)
                assert np.all(np.abs(S2 - S) <= 1e-13 * S)
        oo = np.array([0, outer - 1, outer // 2])
        ii = np.array([inner - 1, 0, inner // 2])
        m1, s1 = orc.softmax_denom_dim_at(x, outer, R, inner, oo, ii)
        assert np.array_equal(m1, M[oo, ii]) and np.array_equal(s1, S[oo, ii])


def pin_softmax_special(orc):
    """IEEE special cases, checked against torch.logsumexp in float64 (which
    also shifts by 0 where the maximum is infinite): -Inf terms add nothing,
    an all -Inf column gives (-Inf, 0), a +Inf term gives (+Inf, +Inf), a NaN
    gives NaN."""
    import torch
    inf, nan = math.inf, math.nan
    cols = [[-inf, -inf, -inf], [1.0, -inf, 2.0], [-inf, 5.0, -inf], [inf, 1.0, -2.0],
            [inf, -inf, 0.0], [inf, inf, 3.0], [nan, 1.0, 2.0], [1.0, 2.0, nan],
            [-inf, nan, inf], [-0.0, -0.0, -0.0], [-30.0, 0.0, -0.0]]
    x = np.array(cols, np.float32).T.copy()      # [R = 3, inner = len(cols)]
    M, S = orc.softmax_denom_dim(x, 1, 3, len(cols))
    M, S = M.reshape(-1), S.reshape(-1)
    lse = torch.logsumexp(torch.from_numpy(x.astype(np.float64)), dim=0).numpy()
    with np.errstate(divide="ignore", invalid="ignore"):
        ours = np.where(np.isfinite(M), M, 0.0) + np.log(S)
    for j, col in enumerate(cols):
        if math.isnan(lse[j]):
            assert math.isnan(M[j]) and math.isnan(S[j]), col
        elif math.isinf(lse[j]):
            assert ours[j] == lse[j], (col, M[j], S[j])
        else:
            assert abs(ours[j] - lse[j]) <= 1e-15 * (1 + abs(lse[j])), (col, M[j], S[j])
    assert M[0] == -inf and S[0] == 0.0
    assert S[1] == 1.0 + math.exp(-1.0) and M[1] == 2.0
    assert M[2] == 5.0 and S[2] == 1.0
    assert M[3] == inf and S[3] == inf
    assert M[9] == 0.0 and S[9] == 3.0


ALL_PINS = [
    pin_harmonic, pin_constants_1d, pin_integers_1d, pin_fsum_1d,
    pin_special_values_1d, pin_index_closed_form, pin_constants_axis,
    pin_bruteforce_axis, pin_fsum_axis, pin_special_values_axis,
    pin_page_shape_facts, pin_sumsq_closed_form, pin_sumsq_exact_and_fsum,
    pin_max_min_library, pin_max_min_special, pin_cumsum_page_example,
    pin_cumsum_library, pin_cumsum_fsum, pin_softmax_constants, pin_softmax_geometric,
    pin_softmax_library, pin_softmax_special,
]
