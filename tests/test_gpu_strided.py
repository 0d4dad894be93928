"""GPU parity of reductions over strided views (rd_reduce_strided), against
the oracle run on a contiguous copy of the same view.

Integer data makes every summation order exact, so each result must equal
the oracle's bit for bit.  The views cover each path the planner takes for
a view: columns with a row stride (slices, every other row, broadcast rows
of stride 0), rows with a row stride (slices, broadcast), a transposed
array read as columns or as rows, and layouts with no unit stride (the
lane-per-output kernel), each at base offsets 0-3 floats and with forced
kernel shapes and splits.
"""
import numpy as np
import pytest

import oracle
import sum_reduction_amd as rd
import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

OPS = ("sum", "sumsq", "max", "min")


@pytest.fixture(autouse=True)
def _clear_tuning():
    rd.rd_tune_set(None)
    yield
    rd.rd_tune_set(None)


# (name, base length, outer, R, inner, so, sr, si, expected path)
VIEWS = [
    ("transpose_dim1", 257 * 300, 300, 257, 1, 1, 300, 1, "cols"),
    ("transpose_dim0", 257 * 300, 1, 300, 257, 0, 1, 300, "rows"),
    ("row_slice", 500 * 300, 500, 98, 1, 300, 1, 1, "rows"),
    ("short_row_slice", 500 * 300, 500, 40, 1, 300, 1, 1, "rows_short"),
    ("long_row_slice", 20 * 5000, 20, 4493, 1, 5000, 1, 1, "rows"),
    ("inner_slice_small", 8 * 64 * 100, 8, 64, 4, 6400, 100, 1, "cols_small"),
    ("inner_slice_3", 8 * 64 * 100, 8, 64, 3, 6400, 100, 1, "cols_small"),
    ("inner_slice_17", 8 * 64 * 100, 8, 64, 17, 6400, 100, 1, "cols_small"),
    ("inner_slice_wide", 2 * 64 * 3000, 2, 64, 1000, 64 * 3000, 3000, 1, "cols"),
    ("every_other_row", 600 * 700, 1, 300, 700, 0, 1400, 1, "cols"),
    ("broadcast_rows", 300, 1, 50, 300, 0, 0, 1, "cols"),
    ("broadcast_row_sums", 300, 50, 300, 1, 0, 1, 1, "rows"),
    ("rows_of_columns", 6 * 400 * 7, 6, 400, 7, 2800, 1, 400, "rows"),
    ("every_third_column", 200 * 90, 1, 100, 30, 0, 180, 3, "strided"),
    # the kept inner axis 2..32 floats apart and a wide span: the column
    # kernel over the dense span of each row, every si-th column kept
    ("every_third_column_wide", 200 * 900, 1, 100, 300, 0, 1800, 3, "cols"),
    ("every_fifth_3d", 4 * 50 * 1000, 4, 50, 200, 50 * 1000, 1000, 5, "cols"),
    ("every_other_column_rows", 300 * 700, 1, 300, 350, 0, 700, 2, "cols"),
    ("every_32nd_column", 64 * 32 * 200, 1, 64, 200, 0, 32 * 200, 32, "cols"),
    ("every_33rd_column", 64 * 33 * 200, 1, 64, 200, 0, 33 * 200, 33, "strided"),
    ("every_seventh_split", 2 * 3000 * 1400, 2, 3000, 200, 3000 * 1400, 1400, 7, "cols"),
    ("permuted_3d", 5 * 6 * 7, 7, 5, 6, 1, 42, 7, "strided"),
    ("strided_long", 3 * 20000 * 2, 3, 20000, 2, 1, 6, 3, "strided"),
]


def _view_host(base, outer, R, inner, so, sr, si, off):
    v = np.lib.stride_tricks.as_strided(base[off:], shape=(outer, R, inner),
                                        strides=(4 * so, 4 * sr, 4 * si), writeable=False)
    return np.ascontiguousarray(v)


def _data(n, seed, op):
    return workloads.small_ints(n, seed, -2, 2) if op == "sumsq" else workloads.small_ints(n, seed)


def _run(op, views, offsets, seed, tag):
    lib = rd.load()
    cases = [(v, off) for v in views for off in offsets]
    hosts, devs = [], []
    slots = H.OutSlots([v[2] * v[4] for v, _ in cases])
    H.say("%s %s: %d calls of rd_reduce_strided" % (tag, op, len(cases)))
    for k, ((name, n, o, R, i, so, sr, si, _), off) in enumerate(cases):
        base = _data(n + 4, seed + k, op)
        dev = H.upload(base)
        hosts.append(base)
        devs.append(dev)
        st = lib.rd_reduce_strided(dev.data_ptr() + 4 * off, o, R, i, so, sr, si, rd.OPS[op],
                                   slots.ptr(k), H.stream_handle())
        assert st == 0, (name, off, rd.rd_status_string(st))
    outs = slots.fetch()
    for k, ((name, n, o, R, i, so, sr, si, _), off) in enumerate(cases):
        S, _ = oracle.reduce_dim(_view_host(hosts[k], o, R, i, so, sr, si, off), o, R, i, op,
                                 threads=1)
        H.assert_bitwise_equal_oracle(outs[k], S, "%s %s %s off=%d" % (tag, op, name, off))


def test_view_paths():
    for name, n, o, R, i, so, sr, si, path in VIEWS:
        got = rd.rd_plan_strided(256, o, R, i, so, sr, si).as_dict()["path"]
        assert got == path, (name, got, path)


@pytest.mark.parametrize("op", OPS)
def test_views_default_plan(op):
    _run(op, VIEWS, [0, 1, 2, 3], 900 + rd.OPS[op], "views")


VIEW_COLS = [v for v in VIEWS if v[-1] in ("cols", "cols_small")]
VIEW_ROWS = [v for v in VIEWS if v[-1] == "rows"]


@pytest.mark.parametrize("split", [1, 3])
def test_views_forced_column_shapes(split):
    wide = [v for v in VIEW_COLS if v[4] >= 4]
    for cw in (1, 2, 4, 8):
        with rd.tuning(col_waves=cw, row_waves=1, unroll=4, split=split, path=4):
            _run("sum", wide, [0, 3], 910 + cw, "cols cw%d s%d" % (cw, split))
    small = [v for v in VIEW_COLS if v[-1] == "cols_small"]
    with rd.tuning(unroll=4, split=split, path=5):
        _run("max", small, [0, 1], 915, "cols_small s%d" % split)


@pytest.mark.parametrize("group,unroll", [(64, 8), (256, 16)])
def test_views_forced_row_shapes(group, unroll):
    for split in (1, 3):
        with rd.tuning(group=group, unroll=unroll, split=split):
            _run("sum", VIEW_ROWS, [0, 2], 920 + group + split, "rows g%d p%d" % (group, split))
            _run("min", VIEW_ROWS, [1], 925 + group + split, "rows g%d p%d" % (group, split))


def test_contiguous_view_gives_the_same_bits():
    """A contiguous view through rd_reduce_strided is rd_reduce_dim, bit for bit."""
    for outer, R, inner in ((3, 5000, 1), (1, 1_000_003, 1), (4, 1000, 4095), (50, 300, 7)):
        a = workloads.random(outer * R * inner, 930 + R, "normal")
        x = H.upload(a, 1)
        want = rd.rd_reduce_dim(x, outer, R, inner, "sum").cpu().numpy()
        got = rd.rd_reduce_strided(x, outer, R, inner, R * inner, inner, 1, "sum").cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (outer, R, inner)


def test_torch_style_views():
    """rd.reduce on transposed, sliced and expanded torch tensors equals
    torch's own reduction of the same view (integer data: exact)."""
    t = H.torch()
    a = workloads.small_ints(6 * 70 * 8 * 9, 940).reshape(6, 70, 8, 9)
    x = H.upload(a).view(6, 70, 8, 9)
    views = [(x.transpose(0, 1), 1), (x[1:5], 1), (x[:, 3:60], 1), (x[:, ::2], 1),
             (x.permute(3, 0, 1, 2), 0), (x[:, :, 0, 0].t(), 0), (x[:, :, 0, 0].t(), 1),
             (x[:1].expand(5, 70, 8, 9), 0), (x[:1].expand(5, 70, 8, 9), 1),
             (x[:, :, :, 0], 1), (x[..., ::3], 3), (x.flatten(1).t(), 1)]
    for v, d in views:
        for op, f in (("sum", lambda z: z.sum(d)), ("max", lambda z: z.amax(d)),
                      ("min", lambda z: z.amin(d))):
            got = rd.reduce(v, op, d).cpu()
            want = f(v).cpu()
            assert t.equal(got, want), (tuple(v.shape), v.stride(), d, op)
    # no single [outer, R, inner] view: refused, not silently copied
    for v, d in ((x[:, :, :, 2:5], 1), (x.transpose(0, 1), 0), (x.transpose(2, 3), 1)):
        with pytest.raises(ValueError):
            rd.reduce(v, "sum", d)


@pytest.mark.parametrize("split", [1, 2, 7, 40])
def test_views_forced_strided_splits(split):
    """The lane-per-output kernel with R cut into slabs (and their combine)."""
    strided = [v for v in VIEWS if v[-1] == "strided"]
    with rd.tuning(split=split):
        for op in OPS:
            _run(op, strided, [0, 1, 3], 950 + split, "strided s%d" % split)


def test_binding_refuses_views_past_the_storage():
    """rd_reduce_strided from Python checks the view against the tensor's
    storage (an offset view included) before calling the library."""
    t = H.torch()
    x = t.zeros(1000, device="cuda")[10:]          # 990 floats from x's start
    rd.rd_reduce_strided(x, 2, 10, 5, 900, 5, 1)   # last = 900 + 45 + 4 = 949: fine
    with pytest.raises(ValueError):
        rd.rd_reduce_strided(x, 2, 10, 5, 941, 5, 1)   # last = 990: one past
    with pytest.raises(ValueError):
        rd.rd_reduce_strided(x, 2, 10, 5, -1, 5, 1)


def test_softmax_denominator_over_views():
    """rd_softmax_denom_strided on every view: terms 0 / -Inf make both
    outputs exact (bit-exact against the oracle on a contiguous copy); random
    data within 1e-5 * s + 1e-6, maxima exact."""
    lib = rd.load()
    t = H.torch()
    for k, (name, n, o, R, i, so, sr, si, _) in enumerate(VIEWS):
        for kind in ("mask", "normal"):
            if kind == "mask":
                bits = workloads.small_ints(n + 4, 960 + k, 0, 1)
                base = np.where(bits > 0, np.float32(0), np.float32(-np.inf)).astype(np.float32)
            else:
                base = workloads.random(n + 4, 970 + k, "normal") * np.float32(6)
            dev = H.upload(base)
            slots = H.OutSlots([o * i, o * i])
            st = lib.rd_softmax_denom_strided(dev.data_ptr() + 4, o, R, i, so, sr, si,
                                              slots.ptr(0), slots.ptr(1), H.stream_handle())
            assert st == 0, (name, rd.rd_status_string(st))
            gm, gs = slots.fetch()
            M, S = oracle.softmax_denom_dim(_view_host(base, o, R, i, so, sr, si, 1), o, R, i)
            what = "softmax %s %s" % (kind, name)
            H.assert_bitwise_equal_oracle(gm, M, what + " (max)")
            if kind == "mask":
                H.assert_bitwise_equal_oracle(gs, S, what + " (sum)")
            else:
                H.assert_within_tolerance(gs, S, S, what + " (sum)")
    # torch-style: softmax and log-sum-exp from the pair of a transposed view
    a = (workloads.random(300 * 500, 980, "normal") * np.float32(3)).reshape(300, 500)
    x = H.upload(a).view(300, 500)
    for d in (0, 1):
        m, s = rd.softmax_denom(x.t(), d)
        lse = (m + t.log(s)).cpu().numpy()
        ref = t.logsumexp(t.from_numpy(a.T.astype(np.float64)), d).numpy()
        assert np.abs(lse - ref).max() <= 1e-5 * (1 + np.abs(ref).max()), d
