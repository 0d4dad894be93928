"""GPU parity of the cumulative sum (rd_cumsum_dim) against the oracle.

Integer data (ints in [-8, 8]) keeps every running sum exact in fp32, so the
GPU must match the oracle bit for bit, in both directions, for every shape
here: rows around the 4096-element tile, columns around the 4-column lanes,
forced splits into pieces / slabs, misaligned bases, in place.  Random data
at the problem-91 size: every output within 1e-5 * (sum of |x| over its
terms) + 1e-6, repeats bitwise identical.
"""
import numpy as np
import pytest

import oracle
import sum_reduction_amd as rd
import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _clear_tuning():
    rd.rd_tune_set(None)
    yield
    rd.rd_tune_set(None)


def _sweep(shapes, offsets, seed, tag, reverse_modes=(True, False)):
    maxn = max(o * r * i for o, r, i in shapes)
    data = workloads.small_ints(maxn + max(offsets) + 1, seed)
    dev = H.upload(data)
    lib = rd.load()
    cases = [(s, off, rev) for s in shapes for off in offsets for rev in reverse_modes]
    slots = H.OutSlots([o * r * i for (o, r, i), _, _ in cases])
    H.say("%s: %d calls of rd_cumsum_dim" % (tag, len(cases)))
    for k, ((o, r, i), off, rev) in enumerate(cases):
        x = dev[off:off + o * r * i]
        st = lib.rd_cumsum_dim(x.data_ptr() if x.numel() else None, o, r, i, int(rev),
                               slots.ptr(k), H.stream_handle())
        assert st == 0, ((o, r, i), off, rev, rd.rd_status_string(st))
    outs = slots.fetch()
    for k, ((o, r, i), off, rev) in enumerate(cases):
        S, _ = oracle.cumsum_dim(data[off:off + o * r * i], o, r, i, rev, threads=2)
        H.assert_bitwise_equal_oracle(outs[k], S, "%s shape=%s off=%d rev=%d"
                                      % (tag, (o, r, i), off, rev))


def test_small_shapes():
    shapes = [(o, r, i) for o in range(5) for r in range(6) for i in range(6)]
    _sweep(shapes, [0, 1, 3], 800, "scan small")


def test_rows_around_tiles():
    shapes = [(3, r, 1) for r in (15, 16, 17, 255, 4095, 4096, 4097, 8191, 8192, 12289)]
    shapes += [(300, 5000, 1), (1, 100_003, 1), (2, 65536, 1)]
    _sweep(shapes, [0, 1, 2, 3], 801, "scan rows")


def test_few_rows_one_pass_plans():
    """Few rows that are not cut: a workgroup per row in one pass -- 4 waves
    for rows of 2-4 tiles, 8 past 16384 positions, 16 from 65536 -- up to
    the longest rows the planner leaves uncut (fewer rows than a third of
    the CUs take the look-back from 65536 positions on)."""
    shapes = [(40, 16384, 1), (5, 16385, 1), (86, 65536, 1), (2, 65535, 1),
              (86, 131072, 1), (300, 4097, 1)]
    for (o, r, i), group in zip(shapes, (256, 512, 1024, 512, 1024, 256)):
        p = rd.rd_plan_cumsum(256, o, r, i)
        assert (p.split, p.group, p.passes) == (1, group, 1), ((o, r, i), p.as_dict())
    _sweep(shapes, [0, 1], 802, "scan few rows")


@pytest.mark.parametrize("path", [0, 7, 8], ids=["default", "scan_cols", "scan_cols_small"])
def test_columns(path):
    """inner > 1 on both column kernels: 4 columns a lane and 256 a wave
    (scan_cols), or 64/LC rows a load instruction scanned across the wave
    (scan_cols_small, LC = ceil(inner/4) lane-columns per row, inner <= 256)."""
    inners = (2, 3, 4, 5, 7, 8, 12, 17, 31, 32, 33, 63, 64, 65, 100, 128, 129, 255, 256)
    if path != 8:
        inners += (257, 4095)
    shapes = [(o, r, i) for i in inners for (o, r) in ((1, 1), (3, 17), (2, 300))]
    shapes += [(1, 5000, 5), (3, 1000, 4), (2, 777, 2), (1, 4099, 3)]
    if path != 8:
        shapes += [(128, 64, 4095)]
    with rd.tuning(path=path):
        _sweep(shapes, [0, 1, 3], 802 + path, "scan cols path %d" % path)


@pytest.mark.parametrize("split", [1, 2, 3, 7])
def test_forced_splits(split):
    """Rows cut into pieces and columns into slabs: totals, carries, scan."""
    with rd.tuning(split=split):
        _sweep([(1, 3 * 4096 + 5, 1), (3, 20000, 1), (1, 1000, 1), (2, 777, 9), (1, 5000, 4),
                (3, 100, 2), (1, 64, 4095)], [0, 1], 810 + split, "scan split %d" % split)


UNROLLS = [(4, 1, 4), (8, 1, 8), (4, 3, 16), (8, 3, 4), (16, 1, 16), (16, 5, 8)]


@pytest.mark.parametrize("unroll,split,bw", UNROLLS, ids=["u%d_s%d_w%d" % t for t in UNROLLS])
def test_unroll_variants(unroll, split, bw):
    """Rows: 4- and 8-slice chunks (16 is a column-only depth); columns: 4, 8
    and 16 rows per load group and 4, 8, 16 waves a block; around the chunk,
    group and block-width boundaries (tiles of 256 columns)."""
    rows = [(3, r, 1) for r in (1023, 1024, 1025, 2047, 2048, 2049, 3 * 2048 + 7, 5 * 4096 + 1)]
    cols = [(2, r, i) for r in (7, 8, 9, 15, 16, 17, 33, 100) for i in (2, 3, 5, 300)]
    cols += [(2, 37, i) for i in (1023, 1024, 1025, 2049, 4095, 4097)]
    with rd.tuning(unroll=unroll, split=split, col_waves=bw, path=7):
        _sweep(cols, [0, 1], 850 + unroll + split, "scan cols u%d s%d w%d" % (unroll, split, bw))
    if unroll != 16:
        small = [(2, r, i) for r in (63, 64, 65, 255, 256, 257, 600) for i in (2, 3, 4, 9, 40, 128)]
        with rd.tuning(unroll=unroll, split=split, path=8):
            _sweep(small, [0, 1], 855 + unroll + split, "scan small u%d s%d" % (unroll, split))
    if unroll != 16:
        with rd.tuning(unroll=unroll, split=split):
            _sweep(rows, [0, 3], 860 + unroll + split, "scan rows u%d s%d" % (unroll, split))


ROUNDS = [(rw, u) for rw in (2, 4, 8, 16) for u in (4, 8)]


@pytest.mark.parametrize("rw,unroll", ROUNDS, ids=["rw%d_u%d" % t for t in ROUNDS])
def test_columns_by_row_rounds(rw, unroll):
    """Column scans whose block's rw waves take turns on one tile's groups
    of `unroll` rows: R around the round (rw * unroll rows) and group
    boundaries, ragged and partial tiles (inner % 4 != 0, lanes past the
    row's end), several tiles and outer indices."""
    per = rw * unroll
    shapes = [(2, r, i) for r in (1, unroll - 1, unroll, unroll + 1, per - 1, per, per + 1,
                                  2 * per + 3, 3 * per)
              for i in (4, 5, 300)]
    shapes += [(3, 5 * per + 7, 1023), (1, 4 * per, 4095), (2, per + 1, 1025)]
    with rd.tuning(row_waves=rw, unroll=unroll, path=7):
        for o, r, i in shapes[:3]:
            p = rd.rd_plan_cumsum(256, o, r, i)
            assert (p.row_waves, p.col_waves, p.split) == (rw, 1, 1), p.as_dict()
        _sweep(shapes, [0, 1, 3], 870 + rw + unroll, "scan rounds rw%d u%d" % (rw, unroll))


@pytest.mark.parametrize("reverse", [True, False], ids=["reverse", "forward"])
def test_tall_columns_random_data(reverse):
    """A 65536-row column scan in one slab (single-wave blocks walking every
    row), U[0, 1) data: the running sums grow to ~32768, so rounding carried
    down the column is the error that matters; the running sums take one add
    per group of rows, which keeps every output within 1e-5 * (sum of |x|
    over its terms) + 1e-6 (one add per row had reached ~1.4x that here)."""
    o, r, i = 1, 65536, 1024
    data = workloads.random(o * r * i, 890 + int(reverse), "uniform", 0.0, 1.0)
    with rd.tuning(row_waves=1, split=1, path=7):
        p = rd.rd_plan_cumsum(256, o, r, i)
        assert (p.split, p.row_waves, p.unroll) == (1, 1, 16), p.as_dict()
        got = rd.rd_cumsum_dim(H.upload(data), o, r, i, reverse)
    S, A = oracle.cumsum_dim(data, o, r, i, reverse, threads=4)
    H.assert_within_tolerance(got.cpu().numpy().reshape(-1), S.reshape(-1), A.reshape(-1),
                              "tall columns %s" % ("reverse" if reverse else "forward"))


def test_column_slabs_default_plans():
    """Few tiles (fewer than half the CUs): slabs of R whose totals come from
    the column reduction, scanned in row rounds of 8 waves -- or by single
    waves for rows a multiple of 8 KB apart -- from each slab's carry; ragged
    slabs, partial tiles, both directions, every output bit-exact."""
    import torch
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    rounds = [(1, 5000, 4095), (2, 3000, 129), (3, 777, 300), (1, 1000, 10922), (4, 513, 2048)]
    lock = [(1, 4100, 4096), (1, 300, 8192)]
    for o, r, i in rounds + lock:
        p = rd.rd_plan_cumsum(cu, o, r, i)
        assert p.split > 1 and p.passes == 3, ((o, r, i), p.as_dict())
        assert p.row_waves == (1 if (o, r, i) in lock else 8), ((o, r, i), p.as_dict())
    _sweep(rounds + lock, [0, 1, 3], 880, "scan col slabs")


@pytest.mark.parametrize("rw,unroll,split", [(8, 8, 3), (4, 4, 7), (2, 8, 2), (16, 4, 5)],
                         ids=["rw8_u8_s3", "rw4_u4_s7", "rw2_u8_s2", "rw16_u4_s5"])
def test_column_slabs_in_row_rounds(rw, unroll, split):
    """Forced slabs scanned in row rounds: slabs shorter than a round, around
    the round and group boundaries, ragged and partial tiles."""
    per = rw * unroll
    shapes = [(2, r, i) for r in (split, per - 1, per * split + 1, 3 * per * split - 5)
              for i in (4, 5, 300)]
    shapes += [(1, 4 * per * split + 7, 4095), (3, per * split, 1025)]
    with rd.tuning(row_waves=rw, unroll=unroll, split=split, path=7):
        _sweep(shapes, [0, 1], 885 + rw + split, "scan slab rounds rw%d u%d s%d"
               % (rw, unroll, split))


def test_columns_by_row_rounds_default_plans():
    """Shapes whose default plan takes row rounds (between half and twice as
    many tiles as CUs), random data: within tolerance of the oracle, and
    bitwise equal from call to call."""
    t = H.torch()
    for o, r, i in ((1, 3000, 32768), (3, 1500, 16384), (64, 512, 1024)):
        p = rd.rd_plan_cumsum(256, o, r, i)
        assert p.row_waves > 1 and p.split == 1, p.as_dict()
        a = workloads.random(o * r * i, 890 + o, "normal")
        x = H.upload(a, 1)
        for rev in (True, False):
            H.say("scan rounds default plan %s rev=%d" % ((o, r, i), rev))
            got = rd.rd_cumsum_dim(x, o, r, i, rev)
            again = rd.rd_cumsum_dim(x, o, r, i, rev)
            assert t.equal(got.view(t.int32), again.view(t.int32))
            S, A = oracle.cumsum_dim(a, o, r, i, rev)
            H.assert_within_tolerance(got.cpu().numpy().reshape(-1), S.reshape(-1),
                                      A.reshape(-1), "rounds %s rev=%d" % ((o, r, i), rev))


BLOCK_ROWS = [(g, u, s) for g in (256, 512, 1024) for (u, s) in ((4, 1), (4, 3), (8, 1), (8, 7))]


@pytest.mark.parametrize("group,unroll,split", BLOCK_ROWS,
                         ids=["g%d_u%d_s%d" % t for t in BLOCK_ROWS])
def test_rows_by_workgroup(group, unroll, split):
    """The row scan with a workgroup per item (group 256, 512 or 1024: 4, 8 or
    16 waves per chunk of waves x 256 x unroll positions, their totals joined
    in LDS), around the chunk boundaries, with pieces, both directions, and in
    place."""
    rows = [(o, r, 1) for o in (1, 3) for r in (1, 63, 255, 256, 1023, 1025, 4095, 4096,
                                                4097, 8191, 8192, 8193, 3 * 4096 + 5, 20000)]
    rows += [(5, 65537, 1), (2, 1 << 17, 1), (1, 32767, 1), (2, 32769, 1), (2, 98305, 1)]
    tag = "g%d u%d s%d" % (group, unroll, split)
    with rd.tuning(group=group, unroll=unroll, split=split):
        p = rd.rd_plan_cumsum(256, 3, 20000, 1)
        assert p.group == group and p.block_threads == group
        _sweep(rows, [0, 3], 880 + group + unroll + split, "scan rows wg " + tag)
        a = workloads.small_ints(3 * 30001, 890 + group + unroll + split)
        x = H.upload(a)
        rd.rd_cumsum_dim(x, 3, 30001, 1, reverse=True, out=x)
        S, _ = oracle.cumsum_dim(a, 3, 30001, 1, True)
        H.assert_bitwise_equal_oracle(x.cpu().numpy(), S, "wg in place " + tag)


STREAM_ROWS = [(256, 8), (512, 8), (1024, 8), (512, 4)]


@pytest.mark.parametrize("group,unroll", STREAM_ROWS, ids=["g%d_u%d" % t for t in STREAM_ROWS])
def test_rows_streamed_by_persistent_workgroups(group, unroll):
    """Whole rows by persistent workgroups that walk their rows' chunks as one
    stream (order = interleaved): bit-exact against the oracle on integer
    data, bitwise equal to a workgroup per row (the same chunks in the same
    order), in place; rows of less than a chunk, of a chunk, with and without
    a partial chunk, fewer rows than workgroups and a ragged last round."""
    chunk = group // 64 * 256 * unroll
    shapes = [(o, r, 1) for o in (1, 3, 700) for r in (1, 5, chunk - 1, chunk, chunk + 1,
                                                       2 * chunk, 2 * chunk + 3, 3 * chunk - 4)]
    shapes += [(2100, 5, 1), (2100, chunk + 1, 1)]
    shapes = [sh for sh in shapes if sh[0] * sh[1] <= 20_000_000]
    tag = "stream g%d u%d" % (group, unroll)
    with rd.tuning(group=group, unroll=unroll, order=1, split=1):
        p = rd.rd_plan_cumsum(256, 700, 2 * chunk, 1)
        assert p.group == group and p.order == 1 and p.split == 1
        assert p.blocks == min(700, 256 * 16 // (group // 64) * (2 if unroll == 4 else 1))
        _sweep(shapes, [0, 1], 1880 + group + unroll, tag)
    t = H.torch()
    rng = np.random.default_rng(group + unroll)
    for o, r in ((700, 2 * chunk + 3), (5, 3 * chunk - 4)):
        a = rng.standard_normal(o * r).astype(np.float32)
        x = H.upload(a)
        for rev in (True, False):
            with rd.tuning(group=group, unroll=unroll, split=1):
                want = rd.rd_cumsum_dim(x, o, r, 1, rev)
            with rd.tuning(group=group, unroll=unroll, order=1, split=1):
                got = rd.rd_cumsum_dim(x, o, r, 1, rev)
                y = x.clone()
                rd.rd_cumsum_dim(y, o, r, 1, rev, out=y)
            t.cuda.synchronize()
            assert t.equal(got.view(t.int32), want.view(t.int32)), (tag, o, r, rev)
            assert t.equal(y.view(t.int32), want.view(t.int32)), (tag, "in place", o, r, rev)


def test_default_splits():
    """Few long rows or few columns: the planner cuts them itself -- rows
    into look-back pieces, columns into slabs (many slabs: the slab carries
    go one wave per column)."""
    shapes = [(1, 1 << 20, 1), (7, 200_000, 1), (1, 100_000, 4), (2, 50_000, 33),
              (1, 1 << 20, 4), (1, 200_000, 300)]
    for shape in shapes:
        p = rd.rd_plan_cumsum(256, *shape).as_dict()
        want = ("lookback", 1) if shape[2] == 1 else ("pass", 3)
        assert p["split"] > 1 and (p["combine"], p["passes"]) == want, (shape, p)
    assert rd.rd_plan_cumsum(256, 1, 1 << 20, 4).split > 64
    _sweep(shapes, [0], 820, "scan default splits")


def test_many_pieces():
    """Thousands of pieces per row: the carries of the piece totals are scanned
    in 256-total chunks by one wave per row."""
    with rd.tuning(combine=1):  # this row would take the look-back by default
        p = rd.rd_plan_cumsum(256, 1, 1 << 24, 1)
        assert p.split == 4096 and p.passes == 3
        _sweep([(1, 1 << 24, 1)], [0], 870, "scan 4096 pieces")
    with rd.tuning(split=700):
        _sweep([(2, 700 * 4096 + 3, 1), (1, 257 * 4096, 1)], [0, 1], 871, "scan 700 pieces")


def test_repeats_bitwise_equal():
    """Random data, every path and split kind: 5 calls give identical bits
    (the totals, their carries and the scan are summed in a fixed order)."""
    t = H.torch()
    for k, shape in enumerate(((3, 50_000, 1), (1, 1 << 21, 1), (2, 3000, 4095), (1, 200_000, 300),
                               (1, 1 << 20, 4), (64, 1000, 33), (1, 100_000, 2))):
        n = shape[0] * shape[1] * shape[2]
        x = H.upload(workloads.random(n, 880 + k, "normal"))
        for rev in (True, False):
            first = rd.rd_cumsum_dim(x, *shape, reverse=rev)
            for _ in range(4):
                assert t.equal(rd.rd_cumsum_dim(x, *shape, reverse=rev).view(t.int32),
                               first.view(t.int32)), (shape, rev)


def test_in_place():
    t = H.torch()
    for shape in ((3, 10_000, 1), (2, 300, 17), (1, 1 << 18, 1)):
        n = shape[0] * shape[1] * shape[2]
        a = workloads.small_ints(n, 830)
        x = H.upload(a)
        rd.rd_cumsum_dim(x, *shape, reverse=True, out=x)
        S, _ = oracle.cumsum_dim(a, *shape, True)
        H.assert_bitwise_equal_oracle(x.cpu().numpy(), S, "in place %s" % (shape,))


def test_special_values():
    """A NaN or Inf reaches every output whose sum includes it, and no other."""
    a = np.ones((3, 9000), np.float32)
    a[1, 5000] = np.nan
    a[2, 100] = np.inf
    got = rd.rd_cumsum_dim(H.upload(a), 3, 9000, 1, reverse=True).cpu().numpy().reshape(3, 9000)
    assert np.isnan(got[1, :5001]).all() and np.isfinite(got[1, 5001:]).all()
    assert np.isinf(got[2, :101]).all() and np.isfinite(got[2, 101:]).all()
    assert np.array_equal(got[0], np.arange(9000, 0, -1, dtype=np.float32))
    got = rd.rd_cumsum_dim(H.upload(a), 3, 9000, 1, reverse=False).cpu().numpy().reshape(3, 9000)
    assert np.isfinite(got[1, :5000]).all() and np.isnan(got[1, 5000:]).all()


def test_torch_style_cumsum():
    a = workloads.small_ints(4 * 5 * 6, 840).reshape(4, 5, 6)
    x = H.upload(a).view(4, 5, 6)
    for dim in range(3):
        f = rd.cumsum(x, dim).cpu().numpy()
        assert np.array_equal(f, np.cumsum(a.astype(np.int64), dim).astype(np.float32))
        r = rd.cumsum(x, dim, reverse=True).cpu().numpy()
        want = np.flip(np.cumsum(np.flip(a.astype(np.int64), dim), dim), dim)
        assert np.array_equal(r, want.astype(np.float32))


@pytest.mark.slow
def test_problem91_full_size():
    """[32768, 32768] reverse cumulative sum along dim 1, U[0, 1): every
    output against the oracle (in row blocks), 3 repeats bitwise equal."""
    w = workloads.SCAN_WORKLOADS["revcumsum_32768x32768"]
    host = workloads.generate(w)
    x = H.upload(host)
    t = H.torch()
    out = t.empty_like(x)
    rd.rd_cumsum_dim(x, w.outer, w.R, w.inner, reverse=True, out=out)
    got = out.cpu().numpy().reshape(w.outer, w.R)
    for _ in range(3):
        again = rd.rd_cumsum_dim(x, w.outer, w.R, w.inner, reverse=True)
        assert t.equal(again, out)
        del again
    block = 1024
    for o0 in range(0, w.outer, block):
        rows = host[o0 * w.R:(o0 + block) * w.R]
        S, A = oracle.cumsum_dim(rows, block, w.R, 1, True)
        H.assert_within_tolerance(got[o0:o0 + block].reshape(-1), S.reshape(-1), A.reshape(-1),
                                  "problem 91 rows %d.." % o0)


@pytest.mark.slow
def test_columns_full_size():
    """[128, 4096, 4095] along dim 1 (the problem-47 shape) both ways, and a
    small-inner [4096, 4096, 4]: every output against the oracle."""
    t = H.torch()
    for shape, seed in (((128, 4096, 4095), 92), ((4096, 4096, 4), 93)):
        o, r, i = shape
        host = workloads.random(o * r * i, seed, "uniform")
        x = H.upload(host)
        for rev in (True, False):
            H.say("columns full size %s reverse=%d" % (shape, rev))
            got = rd.rd_cumsum_dim(x, o, r, i, reverse=rev).cpu().numpy().reshape(o, r * i)
            blk = max(1, (1 << 24) // (r * i))
            for o0 in range(0, o, blk):
                o1 = min(o, o0 + blk)
                S, A = oracle.cumsum_dim(host[o0 * r * i:o1 * r * i], o1 - o0, r, i, rev)
                H.assert_within_tolerance(got[o0:o1].reshape(-1), S.reshape(-1), A.reshape(-1),
                                          "%s rev=%d outer %d.." % (shape, rev, o0))
        del x
        t.cuda.empty_cache()


LOOK_SHAPES = [(g, k) for g in (256, 512, 1024) for k in (4, 8)]


@pytest.mark.parametrize("group,slices", LOOK_SHAPES, ids=["g%d_k%d" % t for t in LOOK_SHAPES])
def test_rows_lookback(group, slices):
    """Rows in one launch, a workgroup per piece of one block chunk, each
    piece's carry formed from the totals earlier pieces publish: rows of one
    and of several pieces, around the chunk, more pieces than a group of 64
    (group totals), misaligned bases, both directions; integer data, bit for
    bit."""
    L = group // 64 * 256 * slices
    shapes = [(3, 1, 1), (3, 5, 1), (2, 4096, 1), (2, L - 1, 1), (2, L, 1), (2, L + 1, 1),
              (5, 3 * L + 17, 1), (1, 64 * L, 1), (1, 65 * L + 7, 1), (2, 130 * L + 3, 1)]
    with rd.tuning(combine=3, group=group, unroll=slices):
        for o, r, i in shapes:
            p = rd.rd_plan_cumsum(256, o, r, i)
            assert (p.combine, p.split, p.passes, p.rows_per_split) == (3, -(-r // L), 1, L)
        _sweep(shapes, [0, 3], 900 + group + slices, "scan lookback g%d k%d" % (group, slices))


def test_rows_lookback_default_plans():
    """Long rows among few take the look-back by default."""
    shapes = [(1, 1 << 24, 1), (5, (1 << 22) + 3, 1), (16, 1 << 20, 1)]
    for shape in shapes:
        p = rd.rd_plan_cumsum(256, *shape)
        assert p.as_dict()["combine"] == "lookback" and p.group == 1024, (shape, p.as_dict())
    _sweep(shapes, [0, 1], 905, "scan lookback default")


def test_rows_lookback_large_arrays():
    """Arrays of 1 GiB and more take the look-back kernel by default, rows in
    ticket order: whole 32768-position rows (one piece each), and rows with
    a partial last piece of 16384 (8 waves); integer data, bit for bit."""
    shapes = [(8192, 32768, 1), (10_000, 27_000, 1)]
    for (o, r, i), (group, P) in zip(shapes, ((1024, 1), (512, 2))):
        p = rd.rd_plan_cumsum(256, o, r, i)
        assert (p.combine, p.group, p.split) == (3, group, P), p.as_dict()
    _sweep(shapes, [0], 906, "scan lookback large", reverse_modes=(True,))


def test_rows_lookback_stream_buffer_matches_workspace():
    """A look-back scan on a stream with a buffer of its own takes it (its
    totals tagged with the launch's epoch, its ticket set back to 0 by the
    workgroup that draws the last one, nothing zeroed before the launch);
    the per-thread default stream takes a zeroed workspace.  On normal data
    the two give the same bits, call after call of different piece counts and
    both directions on one stream, with single-launch reductions (which
    publish into the same buffer) in between."""
    import ctypes
    t = H.torch()
    lib = rd.load()
    shapes = [(16, 1 << 20, 1), (1, (1 << 24) + 5, 1), (5, 300_001, 1), (3, 5 * 16384 + 9, 1)]
    tunes = [{}, {}, dict(combine=3, group=512), dict(combine=3, group=256, unroll=4)]
    maxn = max(o * r * i for o, r, i in shapes)
    a = workloads.random(maxn, 914, "normal")
    x = H.upload(a)
    cols = (2, 100, 1000)
    sizes = [o * r * i for o, r, i in shapes]
    per_thread = 2  # hipStreamPerThread
    results = {}
    for name, h in (("buffer", H.stream_handle()), ("workspace", per_thread)):
        outs = []
        for rep in range(2):
            for (o, r, i), tune, n in zip(shapes, tunes, sizes):
                with rd.tuning(**tune):
                    p = rd.rd_plan_cumsum(256, o, r, i)
                    assert p.combine == 3, ((o, r, i), p.as_dict())
                    for rev in (True, False):
                        y = t.empty(n, device="cuda")
                        t.cuda.synchronize()
                        assert lib.rd_cumsum_dim(x.data_ptr(), o, r, i, int(rev), y.data_ptr(),
                                                 h) == 0
                        outs.append(y)
                red = t.empty(cols[0] * cols[2], device="cuda")
                assert lib.rd_sum_dim(x.data_ptr(), *cols, red.data_ptr(), h) == 0
                outs.append(red)
        if h == per_thread:
            assert lib.hipStreamSynchronize(ctypes.c_void_p(per_thread)) == 0
        t.cuda.synchronize()
        results[name] = [y.cpu().numpy().view(np.uint32) for y in outs]
    for k, (u, w) in enumerate(zip(results["buffer"], results["workspace"])):
        assert np.array_equal(u, w), k
    k = 0
    for (o, r, i), n in zip(shapes, sizes):   # the first call of each shape: reverse
        S, A = oracle.cumsum_dim(a[:n], o, r, i, True)
        H.assert_within_tolerance(results["buffer"][k].view(np.float32), S, A,
                                  "look-back on the stream buffer %s" % ((o, r, i),))
        k += 3


def test_rows_lookback_special_values():
    """A NaN or Inf crosses pieces by the published totals: it reaches every
    output after it in processing order, in its own row only."""
    R = 5 * 16384 + 9
    a = np.ones((3, R), np.float32)
    a[1, 20000] = np.nan            # in the second of six 16384-position pieces
    a[2, R - 100] = np.inf          # in the last piece
    with rd.tuning(combine=3, group=512):
        fwd = rd.rd_cumsum_dim(H.upload(a), 3, R, 1, reverse=False).cpu().numpy().reshape(3, R)
        rev = rd.rd_cumsum_dim(H.upload(a), 3, R, 1, reverse=True).cpu().numpy().reshape(3, R)
    assert np.array_equal(fwd[0], np.arange(1, R + 1, dtype=np.float32))
    assert np.isfinite(fwd[1, :20000]).all() and np.isnan(fwd[1, 20000:]).all()
    assert np.isfinite(fwd[2, :R - 100]).all() and np.isinf(fwd[2, R - 100:]).all()
    assert np.isnan(rev[1, :20001]).all() and np.isfinite(rev[1, 20001:]).all()
    assert np.isinf(rev[2, :R - 99]).all() and np.isfinite(rev[2, R - 99:]).all()
    assert np.array_equal(rev[0], np.arange(R, 0, -1, dtype=np.float32))


def test_rows_lookback_many_groups():
    """More than 64 group totals before a piece: they are read 64 at a time."""
    shape = (1, 4097 * 16384 + 3, 1)
    with rd.tuning(combine=3, group=512):
        p = rd.rd_plan_cumsum(256, *shape)
        assert p.split == 4098
        _sweep([shape], [0], 910, "scan lookback 65 groups")


def test_rows_lookback_in_place_strided_repeats():
    t = H.torch()
    with rd.tuning(combine=3, group=1024):
        a = workloads.small_ints(3 * 100_000, 911)
        x = H.upload(a)
        rd.rd_cumsum_dim(x, 3, 100_000, 1, reverse=True, out=x)
        S, _ = oracle.cumsum_dim(a, 3, 100_000, 1, True)
        H.assert_bitwise_equal_oracle(x.cpu().numpy(), S, "lookback in place")
        # rows 100_007 floats apart: the first 100_000 of each
        b = workloads.small_ints(3 * 100_007, 912)
        view = H.upload(b).view(3, 100_007)[:, :100_000]
        got = rd.cumsum(view, 1).cpu().numpy()
        S, _ = oracle.cumsum_dim(np.ascontiguousarray(b.reshape(3, 100_007)[:, :100_000]).ravel(),
                                 3, 100_000, 1, False)
        H.assert_bitwise_equal_oracle(got.ravel(), S, "lookback row stride")
        # random data: the carries are summed in a fixed order, so repeats agree
        xr = H.upload(workloads.random(2 * 3_000_000, 913, "normal"))
        for rev in (True, False):
            first = rd.rd_cumsum_dim(xr, 2, 3_000_000, 1, reverse=rev)
            for _ in range(4):
                assert t.equal(rd.rd_cumsum_dim(xr, 2, 3_000_000, 1, reverse=rev).view(t.int32),
                               first.view(t.int32)), rev


_SPIN = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np
import torch
import oracle
import workloads
import sum_reduction_amd as rd
from tests import gpu_helpers as H
o, r, L = 4, 40 * 16384 + 5, 16384
a = workloads.small_ints(o * r, 915)
x = H.upload(a)
S, _ = oracle.cumsum_dim(a, o, r, 1, True)
S = np.asarray(S).reshape(o, r)
with rd.tuning(combine=3, group=512):
    y = rd.rd_cumsum_dim(x, o, r, 1, reverse=True).cpu().numpy().reshape(o, r)
nan_pieces = 0
for i in range(o):
    yr, sr = y[i, ::-1], S[i, ::-1]  # processing order of the reverse sum
    for j in range(0, r, L):
        seg = yr[j:j + L]
        if np.isnan(seg).all():
            nan_pieces += 1
        else:
            assert np.array_equal(seg, sr[j:j + L].astype(np.float32)), (i, j)
    assert not np.isnan(yr[:L]).any()  # a row's first piece waits for nothing
print("spin-ok", nan_pieces)
"""


def test_rows_lookback_wait_limit():
    """Waits bounded from the host: with RD_TEST_SPIN_LIMIT=0 every wait
    polls once.  The kernel still ends, and each piece's outputs are either
    exact or all NaN, never a wrong finite sum.  (The limit is read once per
    process, so this runs in a child process.)"""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, RD_TEST_SPIN_LIMIT="0")
    res = subprocess.run([sys.executable, "-c", _SPIN, root], env=env, capture_output=True,
                         text=True, timeout=240, cwd=root)
    assert res.returncode == 0 and "spin-ok" in res.stdout, res.stdout + res.stderr[-3000:]
    H.say(res.stdout.strip())
