"""GPU parity of the other reductions (sum of squares, maximum, minimum),
through rd_reduce_1d / rd_reduce_dim, against the oracle.

Maximum and minimum are exact, so they must match the oracle bit for bit on
any data.  The sum of squares is bit-exact on small integers (values in
[-2, 2]: every partial sum is an integer below 2^24) and within
1e-5 * sum x^2 + 1e-6 on random data.
"""
import numpy as np
import pytest

import oracle
import sum_reduction_amd as rd
import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

OPS3 = ("sumsq", "max", "min")


@pytest.fixture(autouse=True)
def _clear_tuning():
    rd.rd_tune_set(None)
    yield
    rd.rd_tune_set(None)


def _data(n, seed, op):
    # squares of [-2, 2] stay exact in fp32 sums of up to 4 million terms
    return workloads.small_ints(n, seed, -2, 2) if op == "sumsq" else \
        workloads.small_ints(n, seed)


def _sweep_1d(op, ns, offsets, seed, tag):
    data = _data(max(ns) + max(offsets) + 1, seed, op)
    dev = H.upload(data)
    lib = rd.load()
    cases = [(n, off) for n in ns for off in offsets]
    slots = H.OutSlots([1] * len(cases))
    H.say("%s %s: %d calls of rd_reduce_1d" % (tag, op, len(cases)))
    for k, (n, off) in enumerate(cases):
        x = dev[off:off + n]
        st = lib.rd_reduce_1d(x.data_ptr() if n else None, n, rd.OPS[op], slots.ptr(k),
                              H.stream_handle())
        assert st == 0, (op, n, off, rd.rd_status_string(st))
    outs = slots.fetch()
    for k, (n, off) in enumerate(cases):
        S, _ = oracle.reduce_1d(data[off:off + n], op)
        H.assert_bitwise_equal_oracle(outs[k], [S], "%s %s n=%d off=%d" % (tag, op, n, off))


def _sweep_dim(op, shapes, offsets, seed, tag):
    maxn = max(o * r * i for o, r, i in shapes)
    data = _data(maxn + max(offsets) + 1, seed, op)
    dev = H.upload(data)
    lib = rd.load()
    cases = [(s, off) for s in shapes for off in offsets]
    slots = H.OutSlots([o * i for (o, r, i), _ in cases])
    H.say("%s %s: %d calls of rd_reduce_dim" % (tag, op, len(cases)))
    for k, ((o, r, i), off) in enumerate(cases):
        x = dev[off:off + o * r * i]
        st = lib.rd_reduce_dim(x.data_ptr() if x.numel() else None, o, r, i, rd.OPS[op],
                               slots.ptr(k), H.stream_handle())
        assert st == 0, (op, (o, r, i), off, rd.rd_status_string(st))
    outs = slots.fetch()
    for k, ((o, r, i), off) in enumerate(cases):
        S, _ = oracle.reduce_dim(data[off:off + o * r * i], o, r, i, op, threads=1)
        H.assert_bitwise_equal_oracle(outs[k], S, "%s %s shape=%s off=%d"
                                      % (tag, op, (o, r, i), off))


@pytest.mark.parametrize("op", OPS3)
def test_every_small_n(op):
    _sweep_1d(op, list(range(0, 1100)) + [4095, 4096, 4097, 65539, 1_000_003], [0, 1, 2, 3],
              700 + rd.OPS[op], "1d")


@pytest.mark.parametrize("op", OPS3)
def test_small_and_wide_shapes(op):
    shapes = [(o, r, i) for o in range(6) for r in range(6) for i in range(6)]
    shapes += [(o, r, i) for i in (63, 64, 65, 255, 257, 1023, 4095)
               for (o, r) in ((1, 1), (2, 5), (3, 17))]
    shapes += [(1000, 3, 1), (300, 64, 1), (33, 4095, 1), (5, 12289, 1), (2, 4096, 4095),
               (3, 100_003, 1), (5, 37, 2), (3, 1000, 3)]
    _sweep_dim(op, shapes, [0, 1, 3], 710 + rd.OPS[op], "dim")


ROW_SHAPES = [(op, g, u, p, nt, c) for op in OPS3 for (g, u) in ((64, 8), (64, 16), (256, 8),
                                                                  (256, 16))
              for p in (1, 3) for nt in (1, 2) for c in (1, 2) if not (p == 1 and c == 2)]


@pytest.mark.parametrize("op,group,unroll,split,nt,combine", ROW_SHAPES,
                         ids=["%s_g%d_u%d_p%d_nt%d_c%d" % t for t in ROW_SHAPES])
def test_rows_kernel_shapes(op, group, unroll, split, nt, combine):
    with rd.tuning(group=group, unroll=unroll, split=split, nontemporal=nt, combine=combine):
        _sweep_1d(op, [0, 1, 5, 64, 65, 1000, 4097, 65539, 300_007], [0, 3],
                  720 + group + unroll + split, "rows")
        _sweep_dim(op, [(3, 1001, 1), (7, 4099, 1)], [0, 1], 730 + group + unroll, "rows")


COL_SHAPES = [(op, cw, s, nt) for op in OPS3 for cw in (1, 2, 4, 8) for s in (1, 3)
              for nt in (1, 2)]


@pytest.mark.parametrize("op,cw,split,nt", COL_SHAPES,
                         ids=["%s_cw%d_s%d_nt%d" % t for t in COL_SHAPES])
def test_cols_kernel_shapes(op, cw, split, nt):
    shapes = [(1, 1, 4), (2, 5, 4), (3, 17, 5), (2, 33, 63), (1, 64, 64), (2, 7, 65),
              (1, 100, 255), (2, 9, 256), (1, 13, 257), (2, 37, 4095), (1, 19, 4 * 1024 + 3)]
    with rd.tuning(col_waves=cw, row_waves=1, unroll=4, split=split, nontemporal=nt, path=4):
        _sweep_dim(op, shapes, [0, 1, 2, 3], 740 + cw + split, "cols")


# Columns too few for one-wave tiles to give every CU a workgroup: the
# default plan is one tile a block with 8 row waves, in slabs of R (ragged
# last slab, partial tiles, rows of 4095 floats).
SLAB_SHAPES = [(1, 2000, 1000), (3, 777, 300), (1, 5000, 4095), (2, 20000, 129), (1, 300, 130),
               (4, 1031, 2048), (1, 257, 4100), (2, 100, 1000)]


def _device_cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("op", ("sum",) + OPS3)
def test_column_slab_plans(op):
    cu = _device_cus()
    for o, r, i in SLAB_SHAPES:
        p = rd.rd_plan_reduce(cu, o, r, i, op)
        assert (p.col_waves, p.row_waves, p.unroll) == (1, 8, 4), ((o, r, i), p.as_dict())
        assert p.split > 1 and p.blocks <= cu, ((o, r, i), p.as_dict())
    _sweep_dim(op, SLAB_SHAPES, [0, 1, 3], 750 + rd.OPS[op], "cols slabs")


# few slabs of one-wave tiles: the planner joins them in the one launch
ONE_LAUNCH_SHAPES = [(1, 5000, 4095), (1, 300, 130), (4, 1031, 2048), (1, 257, 4100),
                     (2, 100, 1000), (2, 5000, 3000), (1, 200, 4097), (1, 100, 20000)]
ALL_OPS = ("sum",) + OPS3


def _dims_on_stream(dev, cases, op, stream=None):
    """rd_reduce_dim of every (shape, offset) case, one call after another."""
    lib = rd.load()
    slots = H.OutSlots([o * i for (o, r, i), _ in cases])
    for k, ((o, r, i), off) in enumerate(cases):
        x = dev[off:off + o * r * i]
        st = lib.rd_reduce_dim(x.data_ptr(), o, r, i, rd.OPS[op], slots.ptr(k),
                               stream if stream is not None else H.stream_handle())
        assert st == 0, (op, (o, r, i), off, rd.rd_status_string(st))
    return slots.fetch()


@pytest.mark.parametrize("op", ALL_OPS)
def test_column_slabs_one_launch(op):
    """A few slabs of one-wave tiles (at most 16, the grid within the CUs)
    are joined by the last slab's workgroups in the same launch, from results
    the other slabs publish as tagged words: on normal data, bit for bit the
    second kernel's results (combine = 1, the same join order), and against
    the oracle (maximum and minimum exactly, the sums within 1e-5 * sum|x| +
    1e-6).  The calls follow one another on one stream, each finding the
    words of earlier epochs in the buffer."""
    cu = _device_cus()
    for o, r, i in ONE_LAUNCH_SHAPES:
        p = rd.rd_plan_reduce(cu, o, r, i, op)
        assert (p.as_dict()["combine"], p.passes) == ("last_block", 1), ((o, r, i), p.as_dict())
    cases = [(s, off) for s in ONE_LAUNCH_SHAPES for off in (0, 1)]
    maxn = max(o * r * i for o, r, i in ONE_LAUNCH_SHAPES)
    data = workloads.random(maxn + 2, 770 + rd.OPS[op], "normal")
    dev = H.upload(data)
    H.say("column slabs in one launch, %s: %d calls each way" % (op, len(cases)))
    one = _dims_on_stream(dev, cases, op)
    with rd.tuning(combine=1):
        two = _dims_on_stream(dev, cases, op)
    for k, ((o, r, i), off) in enumerate(cases):
        what = "one launch %s shape=%s off=%d" % (op, (o, r, i), off)
        assert np.array_equal(one[k].view(np.uint32), two[k].view(np.uint32)), what
        S, A = oracle.reduce_dim(data[off:off + o * r * i], o, r, i, op, threads=1)
        if op in ("max", "min"):
            H.assert_bitwise_equal_oracle(one[k], S, what)
        else:
            H.assert_within_tolerance(one[k], S, A, what)


def test_column_slabs_one_launch_views():
    """Views read as the dense span of their rows (kept columns 2 and 3
    floats apart) in a plan of a few slabs: the last slab's workgroups keep
    every stride-th column of the words they join; bit for bit the second
    kernel's results, and the oracle's on a contiguous copy of the view."""
    t = H.torch()
    cu = _device_cus()
    base = workloads.random(900 * 6000, 780, "normal")
    dev = H.upload(base).view(900, 6000)
    for rs, cs in ((2, 3), (3, 2), (1, 3)):
        v = dev[::rs, ::cs]
        R, inner = v.shape
        st = (0, v.stride(0), v.stride(1))
        p = rd.rd_plan_strided(cu, 1, R, inner, *st)
        assert p.as_dict()["combine"] == "last_block", ((rs, cs), p.as_dict())
        for op in ALL_OPS:
            one = rd.rd_reduce_strided(dev, 1, R, inner, *st, op=op).cpu().numpy()
            with rd.tuning(combine=1):
                two = rd.rd_reduce_strided(dev, 1, R, inner, *st, op=op).cpu().numpy()
            what = "view [::%d, ::%d] %s" % (rs, cs, op)
            assert np.array_equal(one.view(np.uint32), two.view(np.uint32)), what
            host = v.contiguous().cpu().numpy()
            S, A = oracle.reduce_dim(host, 1, R, inner, op, threads=1)
            if op in ("max", "min"):
                H.assert_bitwise_equal_oracle(one.reshape(1, -1), S, what)
            else:
                H.assert_within_tolerance(one.reshape(1, -1), S, A, what)
    t.cuda.synchronize()


def test_column_slabs_one_launch_streams():
    """Column reduces joined in one launch on four streams at once, 8 calls
    each, exact integer data: each stream's calls use its own buffer."""
    t = H.torch()
    shapes = [(2, 5000, 3000), (1, 257, 4100), (4, 1031, 2048), (1, 100, 20000)]
    maxn = max(o * r * i for o, r, i in shapes)
    data = workloads.small_ints(maxn, 790)
    dev = H.upload(data)
    want = [oracle.sum_dim(data[:o * r * i], o, r, i)[0].astype(np.float32)
            for o, r, i in shapes]
    streams = [t.cuda.Stream() for _ in range(4)]
    outs = []
    t.cuda.synchronize()
    for k in range(32):
        o, r, i = shapes[k % 4]
        with t.cuda.stream(streams[k // 8]):
            outs.append((k % 4, rd.reduce(dev[:o * r * i].view(o, r, i), "sum", 1)))
    t.cuda.synchronize()
    for j, got in outs:
        assert np.array_equal(got.cpu().numpy(), want[j]), shapes[j]


def test_one_launch_fallbacks_match():
    """A stream that gets no buffer of its own -- the per-thread default
    stream (one handle, a different stream in each thread), or streams past
    the 256 a device keeps buffers for -- takes the second kernel for the row
    and column reduces that would otherwise join their partial results in one
    launch: the same bits as calls on a stream with a buffer."""
    import ctypes
    t = H.torch()
    lib = rd.load()
    vp = ctypes.c_void_p
    create, sync, destroy = lib.hipStreamCreate, lib.hipStreamSynchronize, lib.hipStreamDestroy
    create.argtypes, sync.argtypes, destroy.argtypes = [ctypes.POINTER(vp)], [vp], [vp]
    create.restype = sync.restype = destroy.restype = ctypes.c_int
    n, cols = 1_000_003, (2, 100, 1000)
    assert rd.rd_plan_1d(256, n).as_dict()["combine"] == "last_block"
    assert rd.rd_plan_dim(256, *cols).as_dict()["combine"] == "last_block"
    a = workloads.random(n, 797, "normal")
    x = H.upload(a)
    o, r, i = cols
    xc = x[:o * r * i]
    want1 = rd.rd_sum_1d(x).cpu().numpy().view(np.uint32)
    want2 = rd.rd_sum_dim(xc, o, r, i).cpu().numpy().view(np.uint32)
    streams = []
    try:
        for _ in range(300):
            h = vp()
            assert create(ctypes.byref(h)) == 0
            streams.append(h.value)
        per_thread = 2  # hipStreamPerThread
        handles = [per_thread] + streams
        outs = t.empty((len(handles), 1 + o * i), device="cuda")
        t.cuda.synchronize()
        for k, h in enumerate(handles):
            assert lib.rd_sum_1d(x.data_ptr(), n, outs[k].data_ptr(), h) == 0
            assert lib.rd_sum_dim(xc.data_ptr(), o, r, i, outs[k, 1:].data_ptr(), h) == 0
        for h in handles:
            assert sync(h) == 0
        got = outs.cpu().numpy()
    finally:
        for h in streams:
            destroy(h)
    for k in range(len(handles)):
        assert got[k, :1].view(np.uint32)[0] == want1[0], k
        assert np.array_equal(got[k, 1:].view(np.uint32), want2.reshape(-1)), k


def test_split_scratch_streams():
    """Split plans that take a second kernel keep their partial results in
    the scratch of the stream's buffer when they fit: reduces of rows and of
    columns cut into many slabs, and cumulative sums of column slabs, one
    after another on four streams at once (each stream reusing its scratch
    in order), exact integer data, every output against the oracle; the same
    calls on the per-thread default stream (no buffer: the pool) give the
    same bits."""
    import ctypes
    t = H.torch()
    lib = rd.load()
    red = [(64, 262144, 1), (2, 100000, 129), (1, 262144, 512), (3, 100000, 300), (300, 1000, 7)]
    scans = [(1, 5000, 4095), (2, 3000, 129)]
    for o, r, i in red:
        p = rd.rd_plan_dim(256, o, r, i)
        assert p.as_dict()["combine"] == "pass" and 0 < p.workspace_bytes <= 1 << 20, p.as_dict()
    for o, r, i in scans:
        p = rd.rd_plan_cumsum(256, o, r, i)
        assert p.passes == 3 and 0 < p.workspace_bytes <= 1 << 20, p.as_dict()
    maxn = max(o * r * i for o, r, i in red + scans)
    data = workloads.small_ints(maxn, 798)
    x = H.upload(data)
    calls = [("sum", s_) for s_ in red] + [("cumsum", s_) for s_ in scans]
    streams = [t.cuda.Stream() for _ in range(4)]

    def run(handle_of):
        outs = []
        t.cuda.synchronize()
        for k in range(3 * len(calls)):
            kind, (o, r, i) = calls[k % len(calls)]
            y = t.empty(o * i if kind == "sum" else o * r * i, device="cuda")
            h = handle_of(k)
            if kind == "sum":
                st = lib.rd_sum_dim(x.data_ptr(), o, r, i, y.data_ptr(), h)
            else:
                st = lib.rd_cumsum_dim(x.data_ptr(), o, r, i, 0, y.data_ptr(), h)
            assert st == 0, (kind, (o, r, i), rd.rd_status_string(st))
            outs.append(y)
        return outs

    one = run(lambda k: streams[k % 4].cuda_stream)
    t.cuda.synchronize()
    pool = run(lambda k: 2)  # hipStreamPerThread
    assert lib.hipStreamSynchronize(ctypes.c_void_p(2)) == 0
    t.cuda.synchronize()
    for k, (a, b) in enumerate(zip(one, pool)):
        kind, (o, r, i) = calls[k % len(calls)]
        got = a.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), b.cpu().numpy().view(np.uint32)), (kind, o, r, i)
        host = data[:o * r * i]
        S = oracle.sum_dim(host, o, r, i)[0] if kind == "sum" else \
            oracle.cumsum_dim(host, o, r, i, False)[0]
        H.assert_bitwise_equal_oracle(got, S, "scratch %s %s" % (kind, (o, r, i)))


def test_split_scratch_threads_one_stream():
    """Eight host threads make split calls with a second kernel on one shared
    stream (the scratch of its buffer): each call holds the stream's scratch
    from its first launch to its last, so no call's first kernel runs between
    another's two; every result is the oracle's exact integer sum."""
    import threading
    t = H.torch()
    lib = rd.load()
    shapes = [(64, 262144, 1), (2, 100000, 129), (300, 1000, 7)]
    for o, r, i in shapes:
        assert rd.rd_plan_dim(256, o, r, i).as_dict()["combine"] == "pass"
    n = max(o * r * i for o, r, i in shapes)
    data = [workloads.small_ints(n, 800 + k) for k in range(8)]
    xs = [H.upload(a) for a in data]
    want = {(k, s_): oracle.sum_dim(data[k][:s_[0] * s_[1] * s_[2]], *s_)[0].astype(np.float32)
            for k in range(8) for s_ in shapes}
    stream = t.cuda.Stream()
    h = stream.cuda_stream
    outs = {}
    errors = []
    t.cuda.synchronize()

    def work(k):
        try:
            for rep in range(12):
                o, r, i = shapes[(k + rep) % len(shapes)]
                y = t.empty(o * i, device="cuda")
                st = lib.rd_sum_dim(xs[k].data_ptr(), o, r, i, y.data_ptr(), h)
                if st != 0:
                    errors.append((k, rep, st))
                outs[(k, rep)] = ((o, r, i), y)
        except Exception as e:  # reported below
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=work, args=(k,)) for k in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    stream.synchronize()
    for (k, rep), (shape, y) in outs.items():
        assert np.array_equal(y.cpu().numpy(), want[(k, shape)].reshape(-1)), (k, rep, shape)


_COL_PUB_SPIN = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np
import torch
import sum_reduction_amd as rd
import workloads
from tests import gpu_helpers as H
o, R, i = 4, 8192, 2048
assert rd.rd_plan_dim(256, o, R, i).as_dict()["combine"] == "last_block"
a = workloads.small_ints(o * R * i, 795)
x = H.upload(a)
from oracle import sum_dim
want = sum_dim(a, o, R, i)[0].astype(np.float32)
nan = 0
for _ in range(20):
    got = rd.rd_sum_dim(x, o, R, i).cpu().numpy()
    bad = ~((got == want) | np.isnan(got))
    assert not bad.any(), (got[bad][:5], want[bad][:5])
    nan += int(np.isnan(got).sum())
print("col-pub-spin-ok", nan)
"""


def test_column_slabs_one_launch_wait_limit():
    """The last slab's waits bounded from the host: with RD_TEST_SPIN_LIMIT=0
    each unready word is polled once.  Every call ends, each output the
    exact sum or NaN, never a wrong finite value.  (Read once per process:
    a child process.)"""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, RD_TEST_SPIN_LIMIT="0")
    res = subprocess.run([sys.executable, "-c", _COL_PUB_SPIN, root], env=env,
                         capture_output=True, text=True, timeout=240, cwd=root)
    assert res.returncode == 0 and "col-pub-spin-ok" in res.stdout, \
        res.stdout + res.stderr[-3000:]
    H.say(res.stdout.strip())


SMALL = [(op, s, nt) for op in OPS3 for s in (1, 3) for nt in (1, 2)]


@pytest.mark.parametrize("op,split,nt", SMALL, ids=["%s_s%d_nt%d" % t for t in SMALL])
def test_cols_small_kernel_shapes(op, split, nt):
    shapes = [(o, r, i) for i in (2, 3, 4, 5, 8, 17, 63, 64, 100, 128)
              for (o, r) in ((1, 1), (3, 7), (2, 64), (5, 130))]
    with rd.tuning(unroll=4, split=split, nontemporal=nt, path=5):
        _sweep_dim(op, shapes + [(2, 33, 129), (1, 50, 256)], [0, 1, 3], 745 + split + nt,
                   "cols_small")


@pytest.mark.parametrize("op", OPS3)
def test_random_data(op):
    """Non-integer data: max / min bit-exact, sum of squares within tolerance."""
    a = workloads.random(3_000_001, 750, "normal")
    got = rd.rd_reduce_1d(H.upload(a, 1), op).cpu().numpy()
    S, A = oracle.reduce_1d(a, op)
    check = H.assert_bitwise_equal_oracle if op != "sumsq" else None
    if check:
        check(got, [S], "1d " + op)
    else:
        H.assert_within_tolerance(got, [S], [A], "1d " + op)
    for outer, R, inner in ((4, 1000, 4095), (300, 5000, 1), (2, 3000, 3), (64, 100, 100)):
        b = workloads.random(outer * R * inner, 751 + R, "uniform", -3.0, 3.0)
        got = rd.rd_reduce_dim(H.upload(b), outer, R, inner, op).cpu().numpy()
        S, A = oracle.reduce_dim(b, outer, R, inner, op)
        if op == "sumsq":
            H.assert_within_tolerance(got, S, A, "dim %s %s" % (op, (outer, R, inner)))
        else:
            H.assert_bitwise_equal_oracle(got, S, "dim %s %s" % (op, (outer, R, inner)))


def test_special_values():
    """IEEE 754-2019 maximum / minimum on the GPU: NaN propagates, -0 < +0,
    the empty reduction gives -Inf / +Inf (0 for the sum of squares), R == 0
    fills the outputs with it."""
    t = H.torch()
    f = lambda *v: H.upload(np.array(v, dtype=np.float32))
    bits = lambda tns: tns.cpu().numpy().view(np.uint32)[0]
    pz, nz = np.float32(0.0).view(np.uint32), np.float32(-0.0).view(np.uint32)
    for v in ((-0.0, 0.0), (0.0, -0.0), (-0.0, 0.0, -0.0, -0.0, 0.0)):
        assert bits(rd.rd_reduce_1d(f(*v), "max")) == pz, v
        assert bits(rd.rd_reduce_1d(f(*v), "min")) == nz, v
    big = np.full(1_000_003, -0.0, np.float32)
    big[777_777] = 0.0
    assert bits(rd.rd_reduce_1d(H.upload(big), "max")) == pz
    big = np.zeros(1_000_003, np.float32)
    big[5] = -0.0
    assert bits(rd.rd_reduce_1d(H.upload(big), "min")) == nz
    for op in OPS3:
        a = np.ones(1_000_003, np.float32)
        a[500_001] = np.nan
        assert np.isnan(rd.rd_reduce_1d(H.upload(a), op).item()), op
    a = np.ones(1_000_003, np.float32)
    a[3] = np.inf
    assert rd.rd_reduce_1d(H.upload(a), "max").item() == np.inf
    a[3] = -np.inf
    assert rd.rd_reduce_1d(H.upload(a), "min").item() == -np.inf
    e = H.upload(np.zeros(0, np.float32))
    assert rd.rd_reduce_1d(e, "max").item() == -np.inf
    assert rd.rd_reduce_1d(e, "min").item() == np.inf
    assert bits(rd.rd_reduce_1d(e, "sumsq")) == pz
    got = rd.rd_reduce_dim(e, 3, 0, 5, "max").cpu().numpy()
    assert (got == -np.inf).all()
    z = np.ones((3, 999, 70), np.float32)
    z[1, 500, 69] = np.nan
    got = rd.rd_reduce_dim(H.upload(z), 3, 999, 70, "min").cpu().numpy()
    assert np.isnan(got[1, 69]) and np.isfinite(np.delete(got.reshape(-1), 139)).all()


@pytest.mark.slow
@pytest.mark.parametrize("op", OPS3)
@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_full_size(name, op):
    """The five workloads at full size, default plan: max / min bit-exact,
    sum of squares within tolerance; 5 repeats bitwise identical."""
    w = workloads.WORKLOADS[name]
    H.say("%s %s: generating" % (name, op))
    host = workloads.generate(w)
    if w.full_reduce:
        S, A = oracle.reduce_1d(host, op)
        S, A = np.array([S]), np.array([A])
    else:
        S, A = oracle.reduce_dim(host, w.outer, w.R, w.inner, op)
    x = H.upload(host)
    del host

    def run():
        if w.full_reduce:
            return rd.rd_reduce_1d(x, op).cpu().numpy().reshape(-1)
        return rd.rd_reduce_dim(x, w.outer, w.R, w.inner, op).cpu().numpy().reshape(-1)

    first = run()
    if op == "sumsq":
        H.assert_within_tolerance(first, S, A, "%s %s" % (name, op))
    else:
        H.assert_bitwise_equal_oracle(first, S, "%s %s" % (name, op))
    for _ in range(5):
        assert np.array_equal(run().view(np.uint32), first.view(np.uint32))
    del x
    H.torch().cuda.empty_cache()


def test_torch_style_reduce():
    a = workloads.small_ints(6 * 7 * 8 * 9, 760).reshape(6, 7, 8, 9)
    x = H.upload(a).view(6, 7, 8, 9)
    for dim in range(4):
        assert np.array_equal(rd.reduce(x, "max", dim).cpu().numpy(), a.max(axis=dim))
        assert np.array_equal(rd.reduce(x, "min", dim).cpu().numpy(), a.min(axis=dim))
        sq = (a.astype(np.int64) ** 2).sum(axis=dim).astype(np.float32)
        assert np.array_equal(rd.reduce(x, "sumsq", dim).cpu().numpy(), sq)
    assert rd.reduce(x, "max").item() == float(a.max())


@pytest.mark.parametrize("combine", [1, 2], ids=["pass", "last_block"])
def test_many_pieces(combine):
    """Tens of thousands of row pieces (most of them empty past the data's
    end): the piece results are joined four per 16-byte load, 16 loads in
    flight per lane, over several rounds and a ragged tail of 1-3 pieces;
    every operator and the softmax pair, bit-exact on integer (0 / -Inf)
    data, with the second pass and with the fused last-workgroup combine."""
    n = (1 << 22) + 7
    pieces = [4095, 4096, 4097, 16385, 65537]
    lib = rd.load()
    for op in ("sum", "sumsq", "max", "min"):
        with rd.tuning(group=256, unroll=16, split=pieces[0], combine=combine):
            assert rd.rd_plan_1d(256, n).split == pieces[0]
        _data_op = _data(n + 1, 760 + rd.OPS[op], op)
        dev = H.upload(_data_op)
        slots = H.OutSlots([1] * len(pieces))
        for k, P in enumerate(pieces):
            with rd.tuning(group=256, unroll=16, split=P, combine=combine):
                st = lib.rd_reduce_1d(dev.data_ptr(), n, rd.OPS[op], slots.ptr(k),
                                      H.stream_handle())
            assert st == 0, (op, P, rd.rd_status_string(st))
        outs = slots.fetch()
        S, _ = oracle.reduce_1d(_data_op[:n], op)
        for k, P in enumerate(pieces):
            H.assert_bitwise_equal_oracle(outs[k], [S], "%s P=%d combine=%d" % (op, P, combine))
    bits = workloads.small_ints(n, 770, 0, 1)
    mask = np.where(bits > 0, np.float32(0), np.float32(-np.inf)).astype(np.float32)
    dev = H.upload(mask)
    slots = H.OutSlots([1, 1] * len(pieces))
    for k, P in enumerate(pieces):
        with rd.tuning(group=256, unroll=16, split=P, combine=combine):
            st = lib.rd_softmax_denom_1d(dev.data_ptr(), n, slots.ptr(2 * k),
                                         slots.ptr(2 * k + 1), H.stream_handle())
        assert st == 0, ("softmax", P, rd.rd_status_string(st))
    outs = slots.fetch()
    M, Ssm = oracle.softmax_denom_dim(mask, 1, n, 1)
    for k, P in enumerate(pieces):
        H.assert_bitwise_equal_oracle(outs[2 * k], M.reshape(-1), "softmax max P=%d" % P)
        H.assert_bitwise_equal_oracle(outs[2 * k + 1], Ssm.reshape(-1), "softmax sum P=%d" % P)
