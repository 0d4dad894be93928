"""GPU parity of the cumulative sum over strided views (rd_cumsum_strided),
against the oracle run on a contiguous copy of the same view.

Integer data (ints in [-8, 8]) keeps every running sum exact in fp32, so each
output must equal the oracle's bit for bit, in both directions.  The views
cover each path the planner takes: rows with a row stride (slices, broadcast
rows, pieces), columns with outer and row strides (slices, every other row,
broadcast), and views with no unit stride along the lanes' side: a
transposed array scanned along its rows (outputs staged through LDS) or its
columns (inputs staged), permuted axes and a strided inner axis (one lane
per column), short and ragged chunks and column blocks, slabs; each at base
offsets 0-3 floats, with the lane-per-column scan also forced on every view
and cut into forced slab counts.
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


# (name, base length, outer, R, inner, so, sr, si, expected path)
VIEWS = [
    ("transpose_rows", 257 * 300, 300, 257, 1, 1, 300, 1, "scan_strided"),
    ("transpose_cols", 257 * 300, 1, 300, 257, 0, 1, 300, "scan_strided"),
    ("row_slice", 500 * 300, 500, 98, 1, 300, 1, 1, "scan_rows"),
    ("long_row_slice", 20 * 5000, 20, 4493, 1, 5000, 1, 1, "scan_rows"),
    ("row_pieces", 2 * 80000, 2, 70001, 1, 80000, 1, 1, "scan_rows"),
    ("inner_slice_small", 8 * 64 * 100, 8, 64, 4, 6400, 100, 1, "scan_cols_small"),
    ("inner_slice_3", 8 * 64 * 100, 8, 64, 3, 6400, 100, 1, "scan_cols_small"),
    ("inner_slice_17", 8 * 64 * 100, 8, 64, 17, 6400, 100, 1, "scan_cols_small"),
    ("inner_slice_wide", 2 * 64 * 3000, 2, 64, 1000, 64 * 3000, 3000, 1, "scan_cols"),
    ("every_other_row", 600 * 700, 1, 300, 700, 0, 1400, 1, "scan_cols"),
    ("column_slabs", 20000 * 400, 1, 20000, 300, 0, 400, 1, "scan_cols"),
    ("broadcast_rows", 300, 1, 50, 300, 0, 0, 1, "scan_cols"),
    ("broadcast_row_scans", 300, 50, 300, 1, 0, 1, 1, "scan_rows"),
    ("rows_of_columns", 6 * 400 * 7, 6, 400, 7, 2800, 1, 400, "scan_strided"),
    ("every_third_column", 200 * 90, 1, 100, 30, 0, 180, 3, "scan_strided"),
    ("permuted_3d", 5 * 6 * 7, 7, 5, 6, 1, 42, 7, "scan_strided"),
    ("strided_long", 3 * 20000 * 2, 3, 20000, 2, 1, 6, 3, "scan_strided"),
    ("transpose_short_rows", 5 * 1000, 1000, 5, 1, 1, 1000, 1, "scan_strided"),
    ("transpose_short_cols", 7 * 300, 1, 7, 300, 0, 1, 7, "scan_strided"),
    ("transpose_every_third", 70 * 900, 300, 70, 1, 3, 900, 1, "scan_strided"),
    # a strided kept inner axis with a wide span, with and without slabs, and
    # transposes with enough columns for several workgroups per CU
    ("every_third_column_wide", 200 * 900, 1, 100, 300, 0, 1800, 3, "scan_strided"),
    ("every_fifth_3d", 4 * 50 * 1000, 4, 50, 200, 50 * 1000, 1000, 5, "scan_strided"),
    ("every_seventh_slabs", 3000 * 1400, 1, 3000, 200, 0, 1400, 7, "scan_strided"),
    ("transpose_rows_wide", 40 * 20000, 20000, 40, 1, 1, 20000, 1, "scan_strided"),
    ("transpose_cols_wide", 40 * 20000, 1, 40, 20000, 0, 1, 40, "scan_strided"),
]


def _span(o, R, i, so, sr, si):
    return (o - 1) * so + (R - 1) * sr + (i - 1) * si + 1


def _view_host(base, outer, R, inner, so, sr, si, off):
    v = np.lib.stride_tricks.as_strided(base[off:], shape=(outer, R, inner),
                                        strides=(4 * so, 4 * sr, 4 * si), writeable=False)
    return np.ascontiguousarray(v)


def _run(views, offsets, seed, tag, reverse_modes=(True, False)):
    lib = rd.load()
    cases = [(v, off, rev) for v in views for off in offsets for rev in reverse_modes]
    hosts, devs = [], []
    slots = H.OutSlots([v[2] * v[3] * v[4] for v, _, _ in cases])
    H.say("%s: %d calls of rd_cumsum_strided" % (tag, len(cases)))
    for k, ((name, n, o, R, i, so, sr, si, _), off, rev) in enumerate(cases):
        assert _span(o, R, i, so, sr, si) <= n, name
        base = workloads.small_ints(n + 4, seed + k)
        dev = H.upload(base)
        hosts.append(base)
        devs.append(dev)
        st = lib.rd_cumsum_strided(dev.data_ptr() + 4 * off, o, R, i, so, sr, si, int(rev),
                                   slots.ptr(k), H.stream_handle())
        assert st == 0, (name, off, rev, rd.rd_status_string(st))
    outs = slots.fetch()
    for k, ((name, n, o, R, i, so, sr, si, _), off, rev) in enumerate(cases):
        S, _ = oracle.cumsum_dim(_view_host(hosts[k], o, R, i, so, sr, si, off), o, R, i, rev,
                                 threads=2)
        H.assert_bitwise_equal_oracle(outs[k], S, "%s %s off=%d rev=%d"
                                      % (tag, name, off, rev))


# Views with no unit stride along the lanes' side and between half a group of
# 64 columns per CU and a chip of single lanes: one pass in row rounds.
ROUND_VIEWS = [
    ("every_third_column_rounds", 300 * 33000, 1, 300, 10922, 0, 33000, 3, "scan_strided"),
    ("every_other_3d_rounds", 4 * 130 * 20000, 4, 130, 9000, 130 * 20000, 20000, 2,
     "scan_strided"),
    ("every_fifth_ragged", 97 * 60000, 1, 97, 11001, 0, 60000, 5, "scan_strided"),
]


def test_row_round_views_default_plan():
    """The default plan of such views is one pass in row rounds (8 waves a
    group of 64 columns here); R around the round and group boundaries via
    the shapes, ragged last column group; bit-exact."""
    for name, n, o, R, i, so, sr, si, _ in ROUND_VIEWS:
        p = rd.rd_plan_cumsum_strided(256, o, R, i, so, sr, si)
        assert p.row_waves in (2, 4, 8) and p.split == 1 and p.passes == 1, (name, p.as_dict())
    _run(ROUND_VIEWS, [0, 3], 960, "strided rounds")


@pytest.mark.parametrize("rw", [2, 4, 8])
def test_row_rounds_forced(rw):
    """Every lane-per-column view of the table in forced row rounds of rw
    waves (rounds of 8*rw rows): short and ragged R, one to many groups."""
    views = [v for v in VIEWS if v[8] == "scan_strided" and v[4] != 1 and v[6] != 1]
    views += [("rounds_edges_%d" % r, 40 * 1000, 3, r, 70, 13000, 40, 3, "scan_strided")
              for r in (2, 7, 8, 8 * rw - 1, 8 * rw, 8 * rw + 1, 2 * 8 * rw + 3)]
    with rd.tuning(path=10, row_waves=rw):
        for name, n, o, R, i, so, sr, si, _ in views:
            p = rd.rd_plan_cumsum_strided(256, o, R, i, so, sr, si)
            assert p.row_waves == rw and p.split == 1, (name, p.as_dict())
        _run(views, [0, 1], 970 + rw, "strided rounds rw%d" % rw)


def test_view_paths():
    for name, n, o, R, i, so, sr, si, path in VIEWS:
        got = rd.rd_plan_cumsum_strided(256, o, R, i, so, sr, si).as_dict()["path"]
        assert got == path, (name, got, path)


def test_views_default_plan():
    _run(VIEWS, [0, 1, 2, 3], 1200, "scan views")


@pytest.mark.parametrize("split", [1, 3, 40])
def test_views_forced_lane_per_column(split):
    """The lane-per-column kernel on every view (those with a unit stride
    too), R cut into forced slab counts (totals, carries, scan)."""
    with rd.tuning(path=10, split=split):
        _run(VIEWS, [0, 3], 1300 + split, "scan_strided s%d" % split)


def test_contiguous_view_gives_the_same_bits():
    """A contiguous view through rd_cumsum_strided is rd_cumsum_dim, bit for bit."""
    for outer, R, inner in ((3, 5000, 1), (1, 300_001, 1), (4, 1000, 4095), (50, 300, 7)):
        a = workloads.random(outer * R * inner, 1400 + R, "normal")
        x = H.upload(a, 1)
        for rev in (True, False):
            want = rd.rd_cumsum_dim(x, outer, R, inner, rev).cpu().numpy().reshape(-1)
            got = rd.rd_cumsum_strided(x, outer, R, inner, R * inner, inner, 1,
                                       rev).cpu().numpy().reshape(-1)
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (
                outer, R, inner, rev)


def test_lane_per_column_random_data():
    """Random data on the lane-per-column kernel: every output within
    1e-5 * (sum of |x| over its terms) + 1e-6 of the oracle."""
    name, n, o, R, i, so, sr, si, _ = VIEWS[0]
    base = workloads.random(n, 1450, "normal")
    x = H.upload(base)
    for rev in (True, False):
        got = rd.rd_cumsum_strided(x, o, R, i, so, sr, si, rev).cpu().numpy().reshape(-1)
        S, A = oracle.cumsum_dim(_view_host(base, o, R, i, so, sr, si, 0), o, R, i, rev)
        H.assert_within_tolerance(got, S.reshape(-1), A.reshape(-1), "random %s rev=%d"
                                  % (name, rev))


def test_in_place_on_own_layout():
    """out == x is accepted where the view is out's own layout."""
    a = workloads.small_ints(2 * 3000 * 5, 1460)
    x = H.upload(a)
    rd.rd_cumsum_strided(x, 2, 3000, 5, 15000, 5, 1, True, out=x)
    S, _ = oracle.cumsum_dim(a, 2, 3000, 5, True)
    H.assert_bitwise_equal_oracle(x.cpu().numpy(), S, "in place view")


def test_torch_style_views():
    """rd.cumsum on transposed, sliced and expanded torch tensors equals
    numpy's cumulative sum of the same view (integer data: exact); the
    result is contiguous in the view's shape."""
    t = H.torch()
    a = workloads.small_ints(6 * 70 * 8 * 9, 1470).reshape(6, 70, 8, 9)
    x = H.upload(a).view(6, 70, 8, 9)
    views = [(x.transpose(0, 1), 1, (1, 0, 2, 3), None), (x[1:5], 1, None, np.s_[1:5]),
             (x[:, 3:60], 1, None, np.s_[:, 3:60]), (x[:, ::2], 1, None, np.s_[:, ::2]),
             (x.permute(3, 0, 1, 2), 0, (3, 0, 1, 2), None),
             (x[:, :, 0, 0].t(), 0, None, None), (x[:, :, 0, 0].t(), 1, None, None),
             (x[:, :, :, 0], 1, None, np.s_[:, :, :, 0]), (x[..., ::3], 3, None, np.s_[..., ::3])]
    for v, d, perm, sl in views:
        if perm is not None:
            host = np.transpose(a, perm)
        elif sl is not None:
            host = a[sl]
        else:
            host = np.ascontiguousarray(a[:, :, 0, 0].T)
        assert tuple(host.shape) == tuple(v.shape)
        for rev in (False, True):
            got = rd.cumsum(v, d, reverse=rev)
            assert got.is_contiguous() and tuple(got.shape) == tuple(v.shape)
            h64 = host.astype(np.int64)
            want = (np.flip(np.cumsum(np.flip(h64, d), d), d) if rev
                    else np.cumsum(h64, d)).astype(np.float32)
            assert np.array_equal(got.cpu().numpy(), want), (tuple(v.shape), v.stride(), d, rev)
    e = x[:1].expand(5, 70, 8, 9)
    got = rd.cumsum(e, 1).cpu().numpy()
    assert np.array_equal(got, np.broadcast_to(np.cumsum(a[:1].astype(np.int64), 1),
                                               (5, 70, 8, 9)).astype(np.float32))
    with pytest.raises(ValueError):
        rd.cumsum(x.transpose(2, 3), 1)     # no single [outer, R, inner] view
    with pytest.raises(ValueError):
        rd.rd_cumsum_strided(x, 2, 10, 5, 30200, 5, 1)  # past x's storage (30240 floats)
    assert t.equal(rd.cumsum(x[:, ::2], 1), rd.cumsum(x[:, ::2].contiguous(), 1))
