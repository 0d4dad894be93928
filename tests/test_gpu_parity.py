"""GPU parity on small and ragged shapes, through the C ABI, against the oracle.

Integer-valued inputs (ints in [-8, 8]) make every partial sum exact in fp32
whatever the order, so the GPU result must equal the oracle's bit for bit: a
dropped, repeated or misplaced element changes a sum by at least 1.  Shapes
span several tiles and ragged tails; every case also runs with the input
starting 0..3 floats past an aligned address, and every output slot is
followed by guard words that must survive.
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


def _sweep_1d(ns, offsets, seed, tag):
    data = workloads.small_ints(max(ns) + max(offsets) + 1, seed)
    dev = H.upload(data)
    cases = [(n, off) for n in ns for off in offsets]
    slots = H.OutSlots([1] * len(cases))
    H.say("%s: %d calls of rd_sum_1d, n in [%d, %d]" % (tag, len(cases), min(ns), max(ns)))
    for k, (n, off) in enumerate(cases):
        st = H.call_1d(dev[off:off + n], slots.ptr(k))
        assert st == 0, (n, off, rd.rd_status_string(st))
    outs = slots.fetch()
    for k, (n, off) in enumerate(cases):
        S, _ = oracle.sum_1d(data[off:off + n])
        H.assert_bitwise_equal_oracle(outs[k], [S], "%s n=%d off=%d" % (tag, n, off))


def _sweep_dim(shapes, offsets, seed, tag):
    maxn = max(o * r * i for o, r, i in shapes)
    data = workloads.small_ints(maxn + max(offsets) + 1, seed)
    dev = H.upload(data)
    cases = [(s, off) for s in shapes for off in offsets]
    slots = H.OutSlots([o * i for (o, r, i), _ in cases])
    H.say("%s: %d calls of rd_sum_dim" % (tag, len(cases)))
    for k, ((o, r, i), off) in enumerate(cases):
        st = H.call_dim(dev[off:off + o * r * i], o, r, i, slots.ptr(k))
        assert st == 0, ((o, r, i), off, rd.rd_status_string(st))
    outs = slots.fetch()
    for k, ((o, r, i), off) in enumerate(cases):
        S, _ = oracle.sum_dim(data[off:off + o * r * i], o, r, i, threads=1)
        H.assert_bitwise_equal_oracle(outs[k], S, "%s shape=%s off=%d" % (tag, (o, r, i), off))


def test_1d_every_n_up_to_4096():
    _sweep_1d(list(range(0, 4097)), [0, 1, 2, 3], 101, "1d n<=4096")


def test_1d_ragged_large():
    ns = [4097, 8191, 65536 + 3, 262144 + 1, 1_000_003, 2_000_001]
    _sweep_1d(ns, [0, 1, 2, 3], 102, "1d ragged")


def test_dim_every_small_shape():
    shapes = [(o, r, i) for o in range(7) for r in range(7) for i in range(7)]
    _sweep_dim(shapes, [0, 1, 2, 3], 103, "dim [0..6]^3")


def test_dim_wide_inner():
    shapes = [(o, r, i) for i in (63, 64, 65, 127, 128, 129, 255, 256, 257, 1023, 1025, 4095)
              for (o, r) in ((1, 1), (2, 5), (3, 17), (1, 64))]
    _sweep_dim(shapes, [0, 1, 2, 3], 104, "dim wide inner")


def test_dim_rows_paths():
    """inner == 1: short rows (lane per row), wave per row, workgroup per row,
    and rows split into pieces when there are few of them."""
    shapes = [(1000, 3, 1), (257, 63, 1), (300, 64, 1), (65, 1000, 1), (33, 4095, 1),
              (9, 4096, 1), (5, 12289, 1), (3, 100_003, 1), (1, 300_001, 1), (2, 65, 1)]
    _sweep_dim(shapes, [0, 1, 2, 3], 105, "dim rows")


def test_dim_problem47_family():
    """The [128, 4096, 4095] dim-1 shape family at reduced outer and R:
    misaligned rows (4095 floats = 16380 B, 12 B past a 16-B boundary) and a
    3-column tail lane, then a split along R when the grid is too small."""
    shapes = [(2, 4096, 4095), (1, 333, 4095), (3, 64, 4095), (2, 100, 4099)]
    _sweep_dim(shapes, [0, 1, 3], 106, "dim problem-47 family")


ROW_TUNES = [(g, u, p, order, nt, c) for g in (64, 256) for u in (2, 4, 8, 16)
             for p in (1, 2, 5) for order in (1, 2) for nt in (1, 2) for c in (1, 2)
             if not (p == 1 and c == 2)]


@pytest.mark.parametrize("group,unroll,split,order,nt,combine", ROW_TUNES,
                         ids=["g%d_u%d_p%d_o%d_nt%d_c%d" % t for t in ROW_TUNES])
def test_rows_kernel_shapes(group, unroll, split, order, nt, combine):
    """Every instantiated rows-kernel shape, both chunk orders, with and
    without the streaming hint, forced splits with both combines."""
    if not rd.rd_tune_supported("rows", group, 0, unroll):
        pytest.skip("shape not built")
    tag = "rows g%d u%d p%d o%d nt%d c%d" % (group, unroll, split, order, nt, combine)
    seed = 200 + group + unroll + split + 7 * order + 11 * nt + 13 * combine
    with rd.tuning(group=group, unroll=unroll, split=split, order=order, nontemporal=nt,
                   combine=combine):
        _sweep_1d([0, 1, 3, 4, 5, 63, 64, 65, 1000, 4097, 65539, 300_007], [0, 1, 2, 3],
                  seed, tag)
        _sweep_dim([(3, 1001, 1), (2, 5, 1), (7, 4099, 1)], [0, 3], seed + 1, tag + " dim")


COL_TUNES = [(cw, rw, u, s, nt) for (cw, rw) in ((1, 1), (1, 2), (1, 4), (1, 8), (1, 16),
                                                 (2, 1), (2, 2), (2, 4), (2, 8), (4, 1),
                                                 (4, 2), (4, 4), (8, 1), (8, 2), (16, 1))
             for u in (2, 4, 8, 16) for s in (1, 3) for nt in (1, 2)]


@pytest.mark.parametrize("cw,rw,unroll,split,nt", COL_TUNES,
                         ids=["cw%d_rw%d_u%d_s%d_nt%d" % t for t in COL_TUNES])
def test_cols_kernel_shapes(cw, rw, unroll, split, nt):
    """Every instantiated column-kernel shape, with and without a split of R
    and the streaming hint."""
    if not rd.rd_tune_supported("cols", cw, rw, unroll):
        pytest.skip("shape not built")
    shapes = [(1, 1, 4), (2, 5, 4), (3, 17, 5), (2, 33, 63), (1, 64, 64), (2, 7, 65),
              (1, 100, 255), (2, 9, 256), (1, 13, 257), (1, 3, 1023), (2, 37, 4095),
              (1, 19, 4 * 1024 + 3)]
    with rd.tuning(col_waves=cw, row_waves=rw, unroll=unroll, split=split, nontemporal=nt,
                   path=4):
        _sweep_dim(shapes, [0, 1, 2, 3], 400 + cw * 100 + rw * 10 + unroll + split + nt,
                   "cols cw%d rw%d u%d s%d nt%d" % (cw, rw, unroll, split, nt))


def _run_1d_many(ns, data_dev, tag):
    slots = H.OutSlots([1] * len(ns))
    for k, n in enumerate(ns):
        assert H.call_1d(data_dev[:n], slots.ptr(k)) == 0, (tag, n)
    return [o.view(np.uint32)[0] for o in slots.fetch()]


def test_fused_combine_matches_second_pass():
    """The last-workgroup combine and the second kernel sum the piece sums in
    the same order: identical bits on random data, for every row kernel
    shape, and correct against the oracle."""
    a = workloads.random(3_000_007, 61, "normal")
    dev = H.upload(a)
    ns = [70, 4097, 65539, 1_000_001, 3_000_007]
    for group in (64, 256):
        for order in (1, 2):
            common = dict(group=group, order=order, unroll=8)
            with rd.tuning(combine=1, **common):
                two = _run_1d_many(ns, dev, "pass")
            with rd.tuning(combine=2, **common):
                one = _run_1d_many(ns, dev, "last block")
                # and again: new epochs, the buffer holding the last call's words
                again = _run_1d_many(ns, dev, "last block again")
            assert two == one == again, (group, order)
    for n, bits in zip(ns, one):
        S, A = oracle.sum_1d(a[:n])
        got = np.array([bits], np.uint32).view(np.float32)
        H.assert_within_tolerance(got, [S], [A], "fused n=%d" % n)


def test_fused_combine_several_rows_and_streams():
    """Split row sums (few long rows) combined by the last workgroup, on
    several streams at once: each stream has a buffer of its own."""
    t = H.torch()
    outer, R = 5, 1_000_003
    a = workloads.small_ints(outer * R, 62)
    dev = H.upload(a)
    S, _ = oracle.sum_dim(a, outer, R, 1)
    want = S.reshape(-1).astype(np.float32)
    streams = [t.cuda.Stream() for _ in range(4)]
    outs = [t.empty(outer, device="cuda") for _ in range(4 * 8)]
    t.cuda.synchronize()
    with rd.tuning(combine=2):
        assert rd.rd_plan_dim(256, outer, R, 1).as_dict()["combine"] == "last_block"
        for k, o in enumerate(outs):
            with t.cuda.stream(streams[k % 4]):
                rd.rd_sum_dim(dev, outer, R, 1, out=o)
    t.cuda.synchronize()
    for o in outs:
        assert np.array_equal(o.cpu().numpy(), want)


def test_single_launch_combine_by_default_epochs():
    """The 1D sums whose pieces the last workgroup combines by default, one
    call after another on one stream, a large one first: each later call
    finds the buffer holding words of earlier epochs (more of them than it
    has pieces) and takes only its own.  Bit for bit the second kernel's
    results."""
    a = workloads.random(2_000_003, 63, "normal")
    dev = H.upload(a)
    ns = [2_000_003, 70_001, 1_000_000, 4097, 2_000_003, 300_000]
    for n in ns:
        p = rd.rd_plan_1d(256, n).as_dict()
        assert p["combine"] == ("last_block" if p["split"] > 1 else "none"), (n, p)
    one = _run_1d_many(ns, dev, "default")
    with rd.tuning(combine=1):
        two = _run_1d_many(ns, dev, "pass")
    assert one == two


def test_single_launch_combine_from_threads():
    """Eight host threads, four streams (two threads on each): every thread
    runs 1D sums of its own size in the single launch, on its stream, and
    checks each against the oracle's exact integer sum.  Calls on one stream
    from two threads take epochs in whatever order they arrive; calls on
    different streams use different buffers."""
    import threading
    t = H.torch()
    streams = [t.cuda.Stream() for _ in range(4)]
    sizes = [1_000_000 + 7919 * k for k in range(8)]
    data = [workloads.small_ints(n, 70 + k) for k, n in enumerate(sizes)]
    want = [float(a.astype(np.int64).sum()) for a in data]
    devs = [H.upload(a) for a in data]
    t.cuda.synchronize()
    errors = []

    def work(k):
        try:
            with t.cuda.stream(streams[k % 4]):
                for _ in range(40):
                    got = rd.rd_sum_1d(devs[k])
                    t.cuda.current_stream().synchronize()
                    if got.item() != want[k]:
                        errors.append((k, got.item(), want[k]))
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append((k, repr(e)))

    for n in sizes:
        assert rd.rd_plan_1d(256, n).as_dict()["combine"] == "last_block"
    threads = [threading.Thread(target=work, args=(k,)) for k in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads)
    assert errors == [], errors[:5]


def test_single_launch_combine_special_values():
    """A NaN or an Inf in one piece reaches the single-launch sum; the
    maximum and minimum keep IEEE 754-2019 semantics through the words."""
    n = 3_000_000
    assert rd.rd_plan_1d(256, n).as_dict()["combine"] == "last_block"
    a = np.ones(n, np.float32)
    a[2_500_000] = np.inf
    assert rd.rd_sum_1d(H.upload(a)).item() == np.inf
    a[100] = -np.inf
    assert np.isnan(rd.rd_sum_1d(H.upload(a)).item())
    b = np.zeros(n, np.float32)
    b[1_234_567] = np.nan
    assert np.isnan(rd.rd_sum_1d(H.upload(b)).item())
    assert np.isnan(rd.reduce(H.upload(b), "max").item())
    c = np.full(n, -1.0, np.float32)
    c[2_999_999] = -0.0
    c[17] = 0.0
    got = rd.reduce(H.upload(c), "max").item()
    assert got == 0.0 and not np.signbit(got)


_PUB_SPIN = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np
import torch
import sum_reduction_amd as rd
from tests import gpu_helpers as H
n = 3_000_000
assert rd.rd_plan_1d(256, n).as_dict()["combine"] == "last_block"
x = H.upload(np.ones(n, np.float32))
got = [rd.rd_sum_1d(x).item() for _ in range(30)]
assert all(g == float(n) or np.isnan(g) for g in got), got
print("pub-spin-ok", sum(bool(np.isnan(g)) for g in got))
"""


def test_single_launch_combine_wait_limit():
    """The last workgroup's waits bounded from the host: with
    RD_TEST_SPIN_LIMIT=0 each unready word is polled once.  Every call ends,
    with the exact sum or NaN, never a wrong finite value.  (Read once per
    process: a child process.)"""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, RD_TEST_SPIN_LIMIT="0")
    res = subprocess.run([sys.executable, "-c", _PUB_SPIN, root], env=env, capture_output=True,
                         text=True, timeout=240, cwd=root)
    assert res.returncode == 0 and "pub-spin-ok" in res.stdout, res.stdout + res.stderr[-3000:]
    H.say(res.stdout.strip())


SMALL_INNERS = [2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128]
SMALL_TUNES = [(u, s, nt) for u in (2, 4, 8) for s in (1, 3) for nt in (1, 2)]


@pytest.mark.parametrize("unroll,split,nt", SMALL_TUNES,
                         ids=["u%d_s%d_nt%d" % t for t in SMALL_TUNES])
def test_cols_small_kernel_shapes(unroll, split, nt):
    """The several-rows-per-load column kernel: every inner up to 128 it
    takes (and 129..256 when forced), row counts around its row phases,
    forced splits of R."""
    shapes = [(o, r, i) for i in SMALL_INNERS for (o, r) in ((1, 1), (3, 7), (2, 64), (5, 130))]
    with rd.tuning(unroll=unroll, split=split, nontemporal=nt, path=5):
        _sweep_dim(shapes + [(2, 33, 129), (3, 17, 200), (1, 50, 256)], [0, 1, 3],
                   600 + unroll + split + nt, "cols_small u%d s%d nt%d" % (unroll, split, nt))


def test_cols_small_default_plans():
    """Small-inner shapes in the planner's own choice, splits included."""
    shapes = [(1, 100_000, 4), (16, 20_000, 7), (2000, 40, 8), (300, 1000, 2), (7, 3000, 3),
              (1, 1 << 18, 64), (40, 500, 100), (9, 9, 128)]
    _sweep_dim(shapes, [0, 2], 650, "cols_small default")


def test_cols_paths_agree():
    """Both column kernels on the same inputs (inner 4..256): within the
    integer data both are exact, so they agree bit for bit."""
    shapes = [(3, 100, 4), (2, 50, 33), (4, 70, 100), (2, 65, 128), (1, 40, 256)]
    maxn = max(o * r * i for o, r, i in shapes)
    data = workloads.small_ints(maxn, 660)
    dev = H.upload(data)
    for o, r, i in shapes:
        x = dev[:o * r * i]
        with rd.tuning(path=4):
            a = rd.rd_sum_dim(x, o, r, i).cpu().numpy()
        with rd.tuning(path=5):
            b = rd.rd_sum_dim(x, o, r, i).cpu().numpy()
        assert np.array_equal(a, b), (o, r, i)


def test_degenerate_shapes():
    """n == 0 writes +0.0; R == 0 writes zeros; outer*inner == 0 writes nothing."""
    t = H.torch()
    out = t.full((3,), float("nan"), device="cuda")
    x = H.upload(np.zeros(0, np.float32))
    assert H.call_1d(x, out.data_ptr()) == 0
    assert H.call_dim(x, 1, 0, 2, out.data_ptr() + 4) == 0
    t.cuda.synchronize()
    got = out.cpu().numpy()
    assert got[0] == 0.0 and not np.signbit(got[0])
    assert got[1] == 0.0 and got[2] == 0.0 and not np.signbit(got[1:3]).any()
    slots = H.OutSlots([0, 0])
    assert H.call_dim(x, 0, 5, 3, slots.ptr(0)) == 0
    assert H.call_dim(x, 4, 5, 0, slots.ptr(1)) == 0
    slots.fetch()  # guards intact


def test_special_values():
    """NaN and Inf propagate to exactly the outputs that contain them; an
    all -0.0 input sums to +0.0."""
    t = H.torch()
    x = np.ones(1_000_003, np.float32)
    cases = []
    a = x.copy(); a[777_777] = np.nan; cases.append(a)
    a = x.copy(); a[5] = np.inf; cases.append(a)
    a = x.copy(); a[5] = np.inf; a[999_999] = -np.inf; cases.append(a)
    cases.append(np.full(100_000, -0.0, np.float32))
    for k, a in enumerate(cases):
        got = rd.rd_sum_1d(H.upload(a)).cpu().numpy()[0]
        S, _ = oracle.sum_1d(a)
        if np.isnan(S):
            assert np.isnan(got), k
        else:
            assert got == S and np.signbit(got) == np.signbit(S), (k, got, S)
    outer, R, inner = 3, 999, 70
    a = np.ones(outer * R * inner, np.float32).reshape(outer, R, inner)
    a[1, 500, 69] = np.nan
    a[2, 0, 3] = -np.inf
    got = rd.rd_sum_dim(H.upload(a), outer, R, inner).cpu().numpy()
    assert np.isnan(got[1, 69]) and got[2, 3] == -np.inf
    mask = np.ones_like(got, bool); mask[1, 69] = False; mask[2, 3] = False
    assert (got[mask] == R).all()


def test_constant_ones_exact():
    """All-ones inputs sum to exactly n (n <= 2^24): every partial is an integer."""
    t = H.torch()
    for n in (1, 4095, 1_000_000, 1 << 24):
        got = rd.rd_sum_1d(t.ones(n, device="cuda")).item()
        assert got == float(n), (n, got)
    got = rd.rd_sum_dim(t.ones(3 * 4096 * 4095, device="cuda"), 3, 4096, 4095)
    assert bool((got == 4096.0).all())
    got = rd.rd_sum_dim(t.ones(7 * 32768, device="cuda"), 7, 32768, 1)
    assert bool((got == 32768.0).all())


def test_address_independence_random():
    """Random data placed 0..3 floats past an aligned address gives the same
    bits: an element's place in the summation does not depend on the address."""
    a = workloads.random(3_000_001, 77, "normal")
    ref = None
    for off in range(4):
        got = rd.rd_sum_1d(H.upload(a, off)).cpu().numpy()
        ref = got if ref is None else ref
        assert got.view(np.uint32)[0] == ref.view(np.uint32)[0], off
    outer, R, inner = 4, 1000, 4095
    b = workloads.random(outer * R * inner, 78, "uniform")
    ref = None
    for off in range(4):
        got = rd.rd_sum_dim(H.upload(b, off), outer, R, inner).cpu().numpy()
        ref = got if ref is None else ref
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), off


_INJECT = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np
import torch
import sum_reduction_amd as rd
from tests import gpu_helpers as H
want = int(sys.argv[2])
x = H.upload(np.ones(1_000_000, np.float32))
slots = H.OutSlots([1])
assert rd.rd_plan_1d(256, 1_000_000).workspace_bytes > 0
st = H.call_1d(x, slots.ptr(0))
assert st == want, (st, want)
out = slots.fetch()[0]
assert out.view(np.uint32)[0] == H.GUARD_BITS
print("inject-ok", st)
"""


def test_failure_injection_leaves_out_untouched():
    """Forced allocation and launch failures return their status codes and
    enqueue nothing.  The library reads the failure switches once per
    process, so each runs in a child process of its own."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for var, status in (("RD_TEST_FAIL_ALLOC", 3), ("RD_TEST_FAIL_LAUNCH", 4)):
        H.say("failure injection: %s" % var)
        env = dict(os.environ, **{var: "1"})
        res = subprocess.run([sys.executable, "-c", _INJECT, root, str(status)], env=env,
                             capture_output=True, text=True, timeout=240, cwd=root)
        assert res.returncode == 0 and "inject-ok %d" % status in res.stdout, (
            var, res.stdout + res.stderr[-3000:])
    # and the library of this process (no switch set) works
    t = H.torch()
    x = H.upload(np.ones(1_000_000, np.float32))
    assert rd.rd_sum_1d(x).item() == 1_000_000.0


def test_torch_style_wrapper():
    t = H.torch()
    a = workloads.small_ints(6 * 7 * 8 * 9, 9).reshape(6, 7, 8, 9)
    x = H.upload(a).view(6, 7, 8, 9)
    for dim in range(4):
        got = rd.sum(x, dim).cpu().numpy()
        want = a.astype(np.int64).sum(axis=dim).astype(np.float32)
        assert np.array_equal(got, want), dim
    assert rd.sum(x).item() == float(a.astype(np.int64).sum())
