"""CPU oracle for the fp32 sum reduction -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The reduction library never does, and
the oracle shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64 accumulation, built with
gcc ``-O2 -fopenmp -ffp-contract=off``).  This module only builds that file
and marshals numpy arrays into it.

What it computes (the plain definition of a sum, see ``oracle.c``):

* ``sum_1d(x)``            -> (S, A) with S = sum x[i], A = sum |x[i]|
  ("High-Performance Reduction Kernels" README: 1D float32 sum reduction).
* ``sum_dim(x, o, R, i)``  -> (S[o, i], A[o, i]) summed over the middle axis of a
  contiguous [outer, R, inner] array (POPCORNBENCH level-1 problem 47 trace,
  "sum over a dimension", reduce_dim = 1).
* ``sum_dim_at(...)``      -> the same for a list of chosen outputs.
* ``reduce_1d / reduce_dim / reduce_dim_at(..., op)`` -> the same for the
  other reductions, op in {"sum", "sumsq", "max", "min"} ("Seven-step
  reduction" page: sum, max, the L2 norm are the same primitive).
* ``cumsum_dim(x, o, R, i, reverse)`` -> (reverse) cumulative sums along the
  middle axis (POPCORNBENCH level-1 problem 91 trace: cumsum of the flipped
  row, flipped back).
* ``softmax_denom_dim(x, o, R, i)`` -> (M, S): per output the maximum M and
  S = sum exp(x - c), c = M when finite else 0, so the softmax denominator is
  exp(c) * S ("Seven-step reduction" page: the softmax denominator is one of
  the reductions it names); ``softmax_denom_dim_at`` for chosen outputs.
* ``within_tolerance``     -> the acceptance rule |got - S| <= 1e-5*A + 1e-6,
  NaN-aware.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-Wall", "-Wextra"]

_default = None


def build(force: bool = True, source: str = SOURCE, library: str = LIBRARY) -> str:
    """Compile ``source`` (default ``oracle.c``) with gcc into ``library``."""
    global _default
    if not force and os.path.exists(library):
        return library
    tmp = library + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, source, "-lm"], check=True)
    os.replace(tmp, library)
    if library == LIBRARY:
        _default = None
    return library


def _as_f32(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.float32:
        raise TypeError("oracle takes float32 input, got %s" % x.dtype)
    return x


class Oracle:
    """The oracle's entry points, bound to one compiled copy of ``oracle.c``."""

    def __init__(self, library: str = LIBRARY):
        lib = ctypes.CDLL(library)
        i64, dp, vp = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.c_void_p
        lib.oracle_sum_1d.argtypes = [vp, i64, dp, dp]
        lib.oracle_sum_1d.restype = None
        lib.oracle_sum_dim.argtypes = [vp, i64, i64, i64, vp, vp, ctypes.c_int]
        lib.oracle_sum_dim.restype = None
        lib.oracle_sum_dim_at.argtypes = [vp, i64, i64, i64, vp, vp, i64, vp, vp]
        lib.oracle_sum_dim_at.restype = None
        lib.oracle_default_threads.argtypes = []
        lib.oracle_default_threads.restype = ctypes.c_int
        ci = ctypes.c_int
        lib.oracle_reduce_1d.argtypes = [vp, i64, ci, dp, dp]
        lib.oracle_reduce_1d.restype = None
        lib.oracle_reduce_dim.argtypes = [vp, i64, i64, i64, ci, vp, vp, ci]
        lib.oracle_reduce_dim.restype = None
        lib.oracle_reduce_dim_at.argtypes = [vp, i64, i64, i64, ci, vp, vp, i64, vp, vp]
        lib.oracle_reduce_dim_at.restype = None
        lib.oracle_cumsum_dim.argtypes = [vp, i64, i64, i64, ci, vp, vp, ci]
        lib.oracle_cumsum_dim.restype = None
        lib.oracle_softmax_denom_dim.argtypes = [vp, i64, i64, i64, vp, vp, ci]
        lib.oracle_softmax_denom_dim.restype = None
        lib.oracle_softmax_denom_dim_at.argtypes = [vp, i64, i64, i64, vp, vp, i64, vp, vp]
        lib.oracle_softmax_denom_dim_at.restype = None
        self.lib = lib
        self.path = library

    def default_threads(self) -> int:
        return int(self.lib.oracle_default_threads())

    def sum_1d(self, x) -> Tuple[float, float]:
        """(S, A): fp64 sum and fp64 sum of magnitudes of a float32 vector."""
        x = _as_f32(x).reshape(-1)
        s = ctypes.c_double()
        a = ctypes.c_double()
        self.lib.oracle_sum_1d(x.ctypes.data, x.size, ctypes.byref(s), ctypes.byref(a))
        return s.value, a.value

    def sum_dim(self, x, outer: int, R: int, inner: int, threads: int = 0):
        """(S, A), each float64 [outer, inner]: sums over the middle axis."""
        x = _as_f32(x).reshape(-1)
        if x.size != outer * R * inner:
            raise ValueError("size %d != %d*%d*%d" % (x.size, outer, R, inner))
        s = np.empty((outer, inner), dtype=np.float64)
        a = np.empty((outer, inner), dtype=np.float64)
        self.lib.oracle_sum_dim(x.ctypes.data, outer, R, inner, s.ctypes.data,
                                a.ctypes.data, int(threads))
        return s, a

    def sum_dim_at(self, x, outer: int, R: int, inner: int, o_idx, i_idx):
        """(S, A) for the outputs (o_idx[k], i_idx[k]), each from the definition."""
        x = _as_f32(x).reshape(-1)
        if x.size != outer * R * inner:
            raise ValueError("size %d != %d*%d*%d" % (x.size, outer, R, inner))
        o_idx = np.ascontiguousarray(o_idx, dtype=np.int64)
        i_idx = np.ascontiguousarray(i_idx, dtype=np.int64)
        if o_idx.shape != i_idx.shape:
            raise ValueError("index arrays differ in shape")
        if o_idx.size and (o_idx.min() < 0 or o_idx.max() >= outer
                           or i_idx.min() < 0 or i_idx.max() >= inner):
            raise IndexError("sample index out of range")
        s = np.empty(o_idx.size, dtype=np.float64)
        a = np.empty(o_idx.size, dtype=np.float64)
        self.lib.oracle_sum_dim_at(x.ctypes.data, outer, R, inner, o_idx.ctypes.data,
                                   i_idx.ctypes.data, o_idx.size, s.ctypes.data,
                                   a.ctypes.data)
        return s, a


    # ---- other reductions: op is "sum", "sumsq", "max" or "min"
    def reduce_1d(self, x, op: str):
        """(S, A) of the full reduce with ``op``."""
        if op == "sum":
            return self.sum_1d(x)
        x = _as_f32(x).reshape(-1)
        s = ctypes.c_double()
        a = ctypes.c_double()
        self.lib.oracle_reduce_1d(x.ctypes.data, x.size, OPS[op], ctypes.byref(s),
                                  ctypes.byref(a))
        return s.value, a.value

    def reduce_dim(self, x, outer: int, R: int, inner: int, op: str, threads: int = 0):
        """(S, A), each float64 [outer, inner], of the axis reduce with ``op``."""
        if op == "sum":
            return self.sum_dim(x, outer, R, inner, threads)
        x = _as_f32(x).reshape(-1)
        if x.size != outer * R * inner:
            raise ValueError("size %d != %d*%d*%d" % (x.size, outer, R, inner))
        s = np.empty((outer, inner), dtype=np.float64)
        a = np.empty((outer, inner), dtype=np.float64)
        self.lib.oracle_reduce_dim(x.ctypes.data, outer, R, inner, OPS[op], s.ctypes.data,
                                   a.ctypes.data, int(threads))
        return s, a

    def reduce_dim_at(self, x, outer: int, R: int, inner: int, op: str, o_idx, i_idx):
        if op == "sum":
            return self.sum_dim_at(x, outer, R, inner, o_idx, i_idx)
        x = _as_f32(x).reshape(-1)
        o_idx = np.ascontiguousarray(o_idx, dtype=np.int64)
        i_idx = np.ascontiguousarray(i_idx, dtype=np.int64)
        if o_idx.size and (o_idx.min() < 0 or o_idx.max() >= outer
                           or i_idx.min() < 0 or i_idx.max() >= inner):
            raise IndexError("sample index out of range")
        s = np.empty(o_idx.size, dtype=np.float64)
        a = np.empty(o_idx.size, dtype=np.float64)
        self.lib.oracle_reduce_dim_at(x.ctypes.data, outer, R, inner, OPS[op],
                                      o_idx.ctypes.data, i_idx.ctypes.data, o_idx.size,
                                      s.ctypes.data, a.ctypes.data)
        return s, a

    # ---- cumulative sum along the middle axis (same shape out)
    def cumsum_dim(self, x, outer: int, R: int, inner: int, reverse: bool = True,
                   threads: int = 0):
        """(S, A), float64 [outer, R, inner]: the (reverse) cumulative sums of
        x and of |x| along the middle axis."""
        x = _as_f32(x).reshape(-1)
        if x.size != outer * R * inner:
            raise ValueError("size %d != %d*%d*%d" % (x.size, outer, R, inner))
        s = np.empty((outer, R, inner), dtype=np.float64)
        a = np.empty((outer, R, inner), dtype=np.float64)
        self.lib.oracle_cumsum_dim(x.ctypes.data, outer, R, inner, int(bool(reverse)),
                                   s.ctypes.data, a.ctypes.data, int(threads))
        return s, a

    # ---- softmax denominator along the middle axis: (max, shifted sum of exp)
    def softmax_denom_dim(self, x, outer: int, R: int, inner: int, threads: int = 0):
        """(M, S), each float64 [outer, inner]: M = max over the middle axis,
        S = sum exp(x - c) with c = M when M is finite, else 0."""
        x = _as_f32(x).reshape(-1)
        if x.size != outer * R * inner:
            raise ValueError("size %d != %d*%d*%d" % (x.size, outer, R, inner))
        m = np.empty((outer, inner), dtype=np.float64)
        s = np.empty((outer, inner), dtype=np.float64)
        self.lib.oracle_softmax_denom_dim(x.ctypes.data, outer, R, inner, m.ctypes.data,
                                          s.ctypes.data, int(threads))
        return m, s

    def softmax_denom_dim_at(self, x, outer: int, R: int, inner: int, o_idx, i_idx):
        """(M, S) for the outputs (o_idx[k], i_idx[k])."""
        x = _as_f32(x).reshape(-1)
        if x.size != outer * R * inner:
            raise ValueError("size %d != %d*%d*%d" % (x.size, outer, R, inner))
        o_idx = np.ascontiguousarray(o_idx, dtype=np.int64)
        i_idx = np.ascontiguousarray(i_idx, dtype=np.int64)
        if o_idx.shape != i_idx.shape:
            raise ValueError("index arrays differ in shape")
        if o_idx.size and (o_idx.min() < 0 or o_idx.max() >= outer
                           or i_idx.min() < 0 or i_idx.max() >= inner):
            raise IndexError("sample index out of range")
        m = np.empty(o_idx.size, dtype=np.float64)
        s = np.empty(o_idx.size, dtype=np.float64)
        self.lib.oracle_softmax_denom_dim_at(x.ctypes.data, outer, R, inner, o_idx.ctypes.data,
                                             i_idx.ctypes.data, o_idx.size, m.ctypes.data,
                                             s.ctypes.data)
        return m, s


# numbering of the reductions (the same as the library's rd_op)
OPS = {"sum": 0, "sumsq": 1, "max": 2, "min": 3}


def default() -> Oracle:
    """The oracle built from ``oracle.c`` (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default


def default_threads() -> int:
    return default().default_threads()


def sum_1d(x):
    return default().sum_1d(x)


def sum_dim(x, outer: int, R: int, inner: int, threads: int = 0):
    return default().sum_dim(x, outer, R, inner, threads)


def sum_dim_at(x, outer: int, R: int, inner: int, o_idx, i_idx):
    return default().sum_dim_at(x, outer, R, inner, o_idx, i_idx)


def reduce_1d(x, op: str):
    return default().reduce_1d(x, op)


def reduce_dim(x, outer: int, R: int, inner: int, op: str, threads: int = 0):
    return default().reduce_dim(x, outer, R, inner, op, threads)


def reduce_dim_at(x, outer: int, R: int, inner: int, op: str, o_idx, i_idx):
    return default().reduce_dim_at(x, outer, R, inner, op, o_idx, i_idx)


def cumsum_dim(x, outer: int, R: int, inner: int, reverse: bool = True, threads: int = 0):
    return default().cumsum_dim(x, outer, R, inner, reverse, threads)


def softmax_denom_dim(x, outer: int, R: int, inner: int, threads: int = 0):
    return default().softmax_denom_dim(x, outer, R, inner, threads)


def softmax_denom_dim_at(x, outer: int, R: int, inner: int, o_idx, i_idx):
    return default().softmax_denom_dim_at(x, outer, R, inner, o_idx, i_idx)


def tolerance(abs_sum):
    """Per-output acceptance bound 1e-5 * A + 1e-6."""
    return 1e-5 * np.asarray(abs_sum, dtype=np.float64) + 1e-6


def within_tolerance(got, S, A) -> np.ndarray:
    """Elementwise pass/fail of |got - S| <= 1e-5*A + 1e-6.

    NaN-aware: an output passes when both sides are NaN; an infinite oracle
    value must be matched exactly (same sign) by ``got``.
    """
    got = np.asarray(got, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    both_nan = np.isnan(got) & np.isnan(S)
    inf = np.isinf(S)
    with np.errstate(invalid="ignore"):
        close = np.abs(got - S) <= tolerance(A)
    inf_ok = inf & (got == S)
    return both_nan | inf_ok | (close & ~inf & ~np.isnan(S))
