"""Seeded random parity on the GPU: shapes, base offsets, operators, tuning
overrides and strided views drawn at random, every result bit-exact against
the oracle on integer data (for the softmax denominator: terms 0 or -Inf,
whose exponentials are exact).  The draws are fixed by the seeds, so a
failure names a reproducible case.
"""
import numpy as np
import pytest

import oracle
import sum_reduction_amd as rd
import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

MAX_ELEMS = 3_000_000


def _size(rng, hi):
    """Sizes spread over orders of magnitude, small ones often."""
    return int(min(hi, np.exp(rng.uniform(0, np.log(hi + 1))))) if rng.random() < 0.9 else int(rng.integers(0, 8))


def _shape(rng):
    while True:
        outer, R, inner = _size(rng, 5000), _size(rng, 300_000), _size(rng, 5000)
        if outer * R * inner <= MAX_ELEMS:
            return outer, R, inner


def _tune(rng, op, inner):
    if rng.random() < 0.5:
        return {}
    opname = "softmax_denom" if op == 4 else [k for k, v in rd.OPS.items() if v == op][0]
    if inner == 1:
        g, u = [(64, 8), (64, 16), (256, 8), (256, 16)][rng.integers(4)]
        t = dict(group=g, unroll=u, split=int(rng.choice([1, 2, 3, 17])),
                 nontemporal=int(rng.integers(1, 3)), combine=int(rng.integers(1, 3)))
        return t if rd.rd_tune_supported("rows", g, 1, u, opname) else {}
    if inner >= 4 and inner <= 256 and rng.random() < 0.3:
        return dict(unroll=4, split=int(rng.choice([1, 2, 5])), path=5)
    if inner >= 4:
        cw = int(rng.choice([1, 2, 4, 8]))
        if rd.rd_tune_supported("cols", cw, 1, 4, opname):
            return dict(col_waves=cw, row_waves=1, unroll=4, split=int(rng.choice([1, 2, 5])),
                        path=4)
    return {}


def _data(n, seed, op):
    if op == 4:
        bits = workloads.small_ints(n, seed, 0, 1)
        return np.where(bits > 0, np.float32(0), np.float32(-np.inf)).astype(np.float32)
    return workloads.small_ints(n, seed, -2, 2) if op == 1 else workloads.small_ints(n, seed)


def _expected(host, o, R, i, op):
    if op == 4:
        return oracle.softmax_denom_dim(host, o, R, i, threads=1)
    return oracle.reduce_dim(host, o, R, i, ["sum", "sumsq", "max", "min"][op], threads=1)[0], None


@pytest.mark.parametrize("seed", range(16))
def test_random_contiguous(seed):
    rng = np.random.default_rng(7000 + seed)
    lib = rd.load()
    for case in range(50):
        o, R, i = _shape(rng)
        op = int(rng.integers(0, 5))
        off = int(rng.integers(0, 4))
        tune = _tune(rng, op, i)
        n = o * R * i
        host = _data(n + off + 1, 7100 + 100 * seed + case, op)
        dev = H.upload(host)
        nout = o * i
        slots = H.OutSlots([nout, nout])
        what = "seed %d case %d shape %s op %d off %d tune %s" % (seed, case, (o, R, i), op, off, tune)
        H.say(what)
        xp = dev.data_ptr() + 4 * off if n else None
        with rd.tuning(**tune):
            if op == 4:
                st = lib.rd_softmax_denom_dim(xp, o, R, i, slots.ptr(0), slots.ptr(1),
                                              H.stream_handle())
            else:
                st = lib.rd_reduce_dim(xp, o, R, i, op, slots.ptr(0), H.stream_handle())
        assert st == 0, (what, rd.rd_status_string(st))
        got_a, got_b = slots.fetch()
        view = host[off:off + n]
        S, S2 = _expected(view, o, R, i, op)
        H.assert_bitwise_equal_oracle(got_a, S, what)
        if op == 4:
            H.assert_bitwise_equal_oracle(got_b, S2, what + " (sum)")


@pytest.mark.parametrize("seed", range(8))
def test_random_strided(seed):
    rng = np.random.default_rng(8000 + seed)
    lib = rd.load()
    for case in range(50):
        while True:
            o, R, i = _size(rng, 300), _size(rng, 3000), _size(rng, 300)
            if o * R * i <= 600_000:
                break
        # strides: each axis 0, 1, the contiguous value, or a random gap
        def pick(contig):
            return int(rng.choice([0, 1, contig, contig + int(rng.integers(1, 9)),
                                   int(rng.integers(1, 40))]))
        si = pick(1)
        sr = pick(max(i, 1) * max(si, 1))
        so = pick(max(R, 1) * max(sr, 1))
        op = int(rng.integers(0, 4))
        off = int(rng.integers(0, 4))
        ext = 0 if o * R * i == 0 else (o - 1) * so + (R - 1) * sr + (i - 1) * si + 1
        host = _data(ext + off + 1, 8100 + 100 * seed + case, op)
        dev = H.upload(host)
        slots = H.OutSlots([o * i])
        what = "seed %d case %d view %s strides %s op %d off %d" % (seed, case, (o, R, i),
                                                                   (so, sr, si), op, off)
        H.say(what)
        xp = dev.data_ptr() + 4 * off if ext else None
        st = lib.rd_reduce_strided(xp, o, R, i, so, sr, si, op, slots.ptr(0), H.stream_handle())
        assert st == 0, (what, rd.rd_status_string(st))
        (got,) = slots.fetch()
        if o * i == 0:
            continue
        v = np.lib.stride_tricks.as_strided(host[off:], shape=(o, R, i),
                                            strides=(4 * so, 4 * sr, 4 * si), writeable=False)
        S, _ = _expected(np.ascontiguousarray(v), o, R, i, op)
        H.assert_bitwise_equal_oracle(got, S, what)


@pytest.mark.parametrize("seed", range(6))
def test_random_strided_cumsum(seed):
    """rd_cumsum_strided on random views, both directions, sometimes with the
    lane-per-column kernel forced and a random slab count; integer data, so
    every prefix is exact and must equal the oracle's bit for bit."""
    rng = np.random.default_rng(8500 + seed)
    lib = rd.load()
    for case in range(40):
        while True:
            o, R, i = _size(rng, 300), _size(rng, 3000), _size(rng, 300)
            if o * R * i <= 600_000:
                break

        def pick(contig):
            return int(rng.choice([0, 1, contig, contig + int(rng.integers(1, 9)),
                                   int(rng.integers(1, 40))]))
        si = pick(1)
        sr = pick(max(i, 1) * max(si, 1))
        so = pick(max(R, 1) * max(sr, 1))
        rev = int(rng.integers(0, 2))
        off = int(rng.integers(0, 4))
        tune = dict(path=10, split=int(rng.choice([1, 2, 7, 50]))) if rng.random() < 0.3 else {}
        n = o * R * i
        ext = 0 if n == 0 else (o - 1) * so + (R - 1) * sr + (i - 1) * si + 1
        host = workloads.small_ints(ext + off + 1, 8600 + 100 * seed + case)
        dev = H.upload(host)
        slots = H.OutSlots([n])
        what = "seed %d case %d view %s strides %s rev %d off %d tune %s" % (
            seed, case, (o, R, i), (so, sr, si), rev, off, tune)
        H.say(what)
        xp = dev.data_ptr() + 4 * off if ext else None
        with rd.tuning(**tune):
            st = lib.rd_cumsum_strided(xp, o, R, i, so, sr, si, rev, slots.ptr(0) if n else None,
                                       H.stream_handle())
        assert st == 0, (what, rd.rd_status_string(st))
        (got,) = slots.fetch()
        if n == 0:
            continue
        v = np.lib.stride_tricks.as_strided(host[off:], shape=(o, R, i),
                                            strides=(4 * so, 4 * sr, 4 * si), writeable=False)
        S, _ = oracle.cumsum_dim(np.ascontiguousarray(v), o, R, i, bool(rev), threads=1)
        H.assert_bitwise_equal_oracle(got, S, what)


@pytest.mark.parametrize("seed", range(8))
def test_random_contiguous_cumsum(seed):
    """rd_cumsum_dim on random contiguous shapes (sizes over orders of
    magnitude, so every plan -- rows, pieces, look-back, columns in lockstep,
    row rounds, slabs of few tiles with their totals from the column
    reduction, small inner -- comes up), both directions, base offsets 0-3,
    sometimes a forced row-round or slab count; integer data, every prefix
    exact and bit for bit the oracle's."""
    rng = np.random.default_rng(9000 + seed)
    lib = rd.load()
    for case in range(30):
        o, R, i = _shape(rng)
        rev = int(rng.integers(0, 2))
        off = int(rng.integers(0, 4))
        tune = {}
        if i >= 4 and rng.random() < 0.3:
            tune = dict(path=7, row_waves=int(rng.choice([2, 4, 8])),
                        unroll=int(rng.choice([4, 8])), split=int(rng.choice([1, 2, 5, 17])))
        n = o * R * i
        host = workloads.small_ints(n + off + 1, 9100 + 100 * seed + case)
        dev = H.upload(host)
        slots = H.OutSlots([n])
        what = "seed %d case %d shape %s rev %d off %d tune %s" % (seed, case, (o, R, i), rev,
                                                                 off, tune)
        H.say(what)
        xp = dev.data_ptr() + 4 * off if n else None
        with rd.tuning(**tune):
            st = lib.rd_cumsum_dim(xp, o, R, i, rev, slots.ptr(0) if n else None,
                                   H.stream_handle())
        assert st == 0, (what, rd.rd_status_string(st))
        (got,) = slots.fetch()
        if n == 0:
            continue
        S, _ = oracle.cumsum_dim(host[off:off + n], o, R, i, bool(rev), threads=2)
        H.assert_bitwise_equal_oracle(got, S, what)
