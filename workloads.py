"""Seeded synthetic inputs for the fp32 sum reduction.

Shared by the tests, the benchmark and the smoke check: the one module that
both the GPU path's callers and the oracle's callers take their inputs from.
It holds no part of the reduction arithmetic -- it only names the workloads
and fills float32 buffers with seeded values.

Workloads (shapes and distributions as the pages and the benchmark spec give
them; the seeds name the stream, the generator is our reading, see below):

=====================  ===============================  =====================
name                   shape / reduce                   values
=====================  ===============================  =====================
harmonic_1e6           1D, n = 1,000,000                x[i] = fl32(1/(i+1))
uniform_1e8            1D, n = 100,000,000              U[-1, 1), seed 42
normal_1e9             1D, n = 1,000,000,000            N(0, 1), seed 7
cols_128x4096x4095     [128, 4096, 4095], reduce dim 1  U[0, 1), seed 1
rows_32768x32768       [32768, 32768], reduce dim 1     N(0, 1), seed 3
=====================  ===============================  =====================

* ``x[i] = 1/(i+1)`` is the synthetic fallback input of the "High-Performance
  Reduction Kernels" README (Layout section).  The fp64 quotient rounded to
  fp32 equals the fp32 quotient (double rounding is innocuous when the wide
  format has at least 2p+2 bits).
* ``[128, 4096, 4095]`` reduced over dim 1 is the problem of the POPCORNBENCH
  level-1 problem 47 trace ("sum over a dimension"); ``[32768, 32768]`` is the
  input shape of the level-1 problem 91 trace, used here for a row sum.

Generator (a reading: the pages name seeds but no generator).  numpy's PCG64
with ``SeedSequence(seed).spawn(k)``: the flat output is cut into fixed chunks
of 2**22 elements and chunk c is filled from the c-th spawned stream.  The bits
depend only on (seed, n, distribution), never on the number of threads that
fill the chunks.  Uniform values come from ``Generator.random(float32)``
(24-bit mantissa grid) mapped affinely to [a, b); for [-1, 1) the map
``2u - 1`` is exact in fp32.  Normal values come from
``Generator.standard_normal(float32)``.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Tuple

import numpy as np

CHUNK = 1 << 22


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: Tuple[int, ...]      # logical shape of the input tensor
    outer: int                  # the reduce viewed as [outer, R, inner]
    R: int
    inner: int
    dist: str                   # "harmonic" | "uniform" | "normal" | "smallint"
    seed: Optional[int] = None
    lo: float = 0.0             # uniform bounds [lo, hi)
    hi: float = 1.0
    full_reduce: bool = False   # True: 1D sum to one scalar

    @property
    def numel(self) -> int:
        return self.outer * self.R * self.inner

    @property
    def in_bytes(self) -> int:
        return 4 * self.numel

    @property
    def out_numel(self) -> int:
        return self.outer * self.inner

    @property
    def algorithmic_bytes(self) -> int:
        """Bytes a reduction must move: every input once, every output once."""
        return 4 * (self.numel + self.out_numel)


WORKLOADS = {
    w.name: w
    for w in (
        Workload("harmonic_1e6", (1_000_000,), 1, 1_000_000, 1, "harmonic",
                 full_reduce=True),
        Workload("uniform_1e8", (100_000_000,), 1, 100_000_000, 1, "uniform",
                 seed=42, lo=-1.0, hi=1.0, full_reduce=True),
        Workload("normal_1e9", (1_000_000_000,), 1, 1_000_000_000, 1, "normal",
                 seed=7, full_reduce=True),
        Workload("cols_128x4096x4095", (128, 4096, 4095), 128, 4096, 4095,
                 "uniform", seed=1, lo=0.0, hi=1.0),
        Workload("rows_32768x32768", (32768, 32768), 32768, 32768, 1, "normal",
                 seed=3),
    )
}

# The reverse cumulative sum of the POPCORNBENCH level-1 problem 91 trace:
# [32768, 32768] along dim 1, torch.rand input (U[0, 1)); the trace names no
# seed, 91 is ours.  A scan, kept apart from the reductions above.
SCAN_WORKLOADS = {
    w.name: w
    for w in (
        Workload("revcumsum_32768x32768", (32768, 32768), 32768, 32768, 1, "uniform",
                 seed=91),
    )
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_random(out: np.ndarray, seed: int, kind: str, lo: float, hi: float):
    n = out.size
    nch = (n + CHUNK - 1) // CHUNK
    streams = np.random.SeedSequence(seed).spawn(nch)

    def fill(c: int):
        g = np.random.Generator(np.random.PCG64(streams[c]))
        sl = out[c * CHUNK:min(n, (c + 1) * CHUNK)]
        if kind == "normal":
            g.standard_normal(dtype=np.float32, out=sl)
        elif kind == "uniform":
            g.random(dtype=np.float32, out=sl)
            if (lo, hi) != (0.0, 1.0):
                sl *= np.float32(hi - lo)
                sl += np.float32(lo)
        elif kind == "smallint":
            # integers in [lo, hi] inclusive, exactly representable
            sl[...] = g.integers(int(lo), int(hi) + 1, size=sl.size,
                                 dtype=np.int32).astype(np.float32)
        else:
            raise ValueError(kind)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nch)))


def harmonic(n: int, out: Optional[np.ndarray] = None) -> np.ndarray:
    """x[i] = fl32(1/(i+1)), i < n."""
    if out is None:
        out = np.empty(n, dtype=np.float32)
    for start in range(0, n, CHUNK):
        stop = min(n, start + CHUNK)
        out[start:stop] = (1.0 / np.arange(start + 1, stop + 1,
                                           dtype=np.float64)).astype(np.float32)
    return out


def random(n: int, seed: int, dist: str, lo: float = 0.0, hi: float = 1.0,
           out: Optional[np.ndarray] = None) -> np.ndarray:
    """n seeded float32 values of distribution ``dist`` (see module doc)."""
    if out is None:
        out = np.empty(n, dtype=np.float32)
    if out.dtype != np.float32 or out.size != n or not out.flags.c_contiguous:
        raise ValueError("out must be a contiguous float32 buffer of n elements")
    _fill_random(out.reshape(-1), seed, dist, lo, hi)
    return out


def small_ints(n: int, seed: int, lo: int = -8, hi: int = 8,
               out: Optional[np.ndarray] = None) -> np.ndarray:
    """Integers in [lo, hi] as float32: every partial sum of fewer than
    2**24 / max(|lo|, |hi|) of them is exact in fp32, in any order."""
    return random(n, seed, "smallint", lo, hi, out)


def generate(w: Workload, out: Optional[np.ndarray] = None) -> np.ndarray:
    """The flat float32 input of workload ``w`` (``w.numel`` elements)."""
    if w.dist == "harmonic":
        return harmonic(w.numel, out)
    return random(w.numel, w.seed, w.dist, w.lo, w.hi, out)
