"""GPU parity of the softmax denominator (rd_softmax_denom_1d / _dim)
against the oracle.

Per output the kernel returns the maximum m, which is exact and must match
the oracle bit for bit, and s = sum exp(x - c) (c = m when finite, else 0),
which must be within 1e-5 * s + 1e-6 of the oracle's fp64 value (all terms
are non-negative, so s is its own magnitude).

Index coverage is tested bit-exactly with data that makes every term exact:
terms 0 and -Inf give exp(0) = 1 and exp(-Inf) = 0, so s is the count of
zeros (exact in fp32 below 2^24) and m is 0, or -Inf when there is none --
a dropped, doubled or misplaced element changes s by 1.  Columns that are
constant along R (a different constant per output) give m = that constant
and s = R exactly.  Rounding is tested on random data of several scales, on
slowly rising columns (the running maximum moves at almost every term) and
at full size.
"""
import numpy as np
import pytest

import oracle
import sum_reduction_amd as rd
import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

SOFTMAX = 4  # rd_op code of the softmax denominator


@pytest.fixture(autouse=True)
def _clear_tuning():
    rd.rd_tune_set(None)
    yield
    rd.rd_tune_set(None)


def _mask(n, seed):
    """0 or -Inf, each with probability 1/2."""
    bits = workloads.small_ints(n, seed, 0, 1)
    return np.where(bits > 0, np.float32(0.0), np.float32(-np.inf)).astype(np.float32)


def _check(gm, gs, M, S, what, exact=False):
    gm = np.asarray(gm, np.float32).reshape(-1)
    gs = np.asarray(gs, np.float32).reshape(-1)
    M = np.asarray(M, np.float64).reshape(-1)
    S = np.asarray(S, np.float64).reshape(-1)
    H.assert_bitwise_equal_oracle(gm, M, what + " (max)")
    if exact:
        H.assert_bitwise_equal_oracle(gs, S, what + " (sum)")
    else:
        H.assert_within_tolerance(gs, S, S, what + " (sum)")


def _sweep_1d(data, ns, offsets, tag, exact):
    dev = H.upload(data)
    lib = rd.load()
    cases = [(n, off) for n in ns for off in offsets]
    slots = H.OutSlots([1] * (2 * len(cases)))
    H.say("%s: %d calls of rd_softmax_denom_1d" % (tag, len(cases)))
    for k, (n, off) in enumerate(cases):
        x = dev[off:off + n]
        st = lib.rd_softmax_denom_1d(x.data_ptr() if n else None, n, slots.ptr(2 * k),
                                     slots.ptr(2 * k + 1), H.stream_handle())
        assert st == 0, (n, off, rd.rd_status_string(st))
    outs = slots.fetch()
    for k, (n, off) in enumerate(cases):
        M, S = oracle.softmax_denom_dim(data[off:off + n], 1, n, 1)
        _check(outs[2 * k], outs[2 * k + 1], M, S, "%s n=%d off=%d" % (tag, n, off), exact)


def _sweep_dim(data, shapes, offsets, tag, exact):
    dev = H.upload(data)
    lib = rd.load()
    cases = [(s, off) for s in shapes for off in offsets]
    sizes = []
    for (o, r, i), _ in cases:
        sizes += [o * i, o * i]
    slots = H.OutSlots(sizes)
    H.say("%s: %d calls of rd_softmax_denom_dim" % (tag, len(cases)))
    for k, ((o, r, i), off) in enumerate(cases):
        x = dev[off:off + o * r * i]
        st = lib.rd_softmax_denom_dim(x.data_ptr() if x.numel() else None, o, r, i,
                                      slots.ptr(2 * k), slots.ptr(2 * k + 1), H.stream_handle())
        assert st == 0, ((o, r, i), off, rd.rd_status_string(st))
    outs = slots.fetch()
    for k, ((o, r, i), off) in enumerate(cases):
        M, S = oracle.softmax_denom_dim(data[off:off + o * r * i], o, r, i, threads=1)
        _check(outs[2 * k], outs[2 * k + 1], M, S, "%s shape=%s off=%d" % (tag, (o, r, i), off),
               exact)


SMALL_SHAPES = ([(o, r, i) for o in range(6) for r in range(6) for i in range(6)]
                + [(o, r, i) for i in (63, 64, 65, 255, 257, 1023, 4095)
                   for (o, r) in ((1, 1), (2, 5), (3, 17))]
                + [(1000, 3, 1), (300, 64, 1), (33, 4095, 1), (5, 12289, 1), (2, 4096, 4095),
                   (3, 100_003, 1), (5, 37, 2), (3, 1000, 3)])


def test_every_small_n_exact():
    ns = list(range(0, 1100)) + [4095, 4096, 4097, 65539, 1_000_003]
    _sweep_1d(_mask(max(ns) + 4, 800), ns, [0, 1, 2, 3], "1d mask", True)


def test_small_and_wide_shapes_exact():
    maxn = max(o * r * i for o, r, i in SMALL_SHAPES)
    _sweep_dim(_mask(maxn + 4, 801), SMALL_SHAPES, [0, 1, 3], "dim mask", True)


def test_constant_columns_exact():
    """x[o, r, i] = k(o, i), a different integer per output (negative, zero,
    positive, large): m = k, s = R, bit-exact."""
    for outer, R, inner in ((3, 7, 5), (2, 4096, 4095), (500, 70, 1), (4, 3000, 2),
                            (1, 100_000, 1), (7, 999, 129)):
        k = workloads.small_ints(outer * inner, 802 + R, -3000, 3000).reshape(outer, 1, inner)
        x = np.broadcast_to(k, (outer, R, inner)).astype(np.float32).reshape(-1)
        m, s = rd.rd_softmax_denom_dim(H.upload(x, 1), outer, R, inner)
        assert np.array_equal(m.cpu().numpy(), k.reshape(outer, inner)), (outer, R, inner)
        assert np.all(s.cpu().numpy() == R), (outer, R, inner)


ROW_SHAPES = [(g, u, p, nt, c) for (g, u) in ((64, 8), (64, 16), (256, 8), (256, 16))
              for p in (1, 3) for nt in (1, 2) for c in (1, 2) if not (p == 1 and c == 2)]


@pytest.mark.parametrize("group,unroll,split,nt,combine", ROW_SHAPES,
                         ids=["g%d_u%d_p%d_nt%d_c%d" % t for t in ROW_SHAPES])
def test_rows_kernel_shapes(group, unroll, split, nt, combine):
    with rd.tuning(group=group, unroll=unroll, split=split, nontemporal=nt, combine=combine):
        ns = [0, 1, 5, 64, 65, 1000, 4097, 65539, 300_007]
        _sweep_1d(_mask(300_011, 810 + group + unroll), ns, [0, 3], "rows mask", True)
        _sweep_1d(workloads.random(300_011, 811 + split, "normal", 0.0, 1.0) * np.float32(20),
                  ns, [0, 3], "rows normal*20", False)
        shapes = [(3, 1001, 1), (7, 4099, 1)]
        _sweep_dim(_mask(7 * 4099 + 2, 812 + unroll), shapes, [0, 1], "rows mask", True)


COL_SHAPES = [(cw, s, nt) for cw in (1, 2, 4, 8) for s in (1, 3) for nt in (1, 2)]


@pytest.mark.parametrize("cw,split,nt", COL_SHAPES, ids=["cw%d_s%d_nt%d" % t for t in COL_SHAPES])
def test_cols_kernel_shapes(cw, split, nt):
    shapes = [(1, 1, 4), (2, 5, 4), (3, 17, 5), (2, 33, 63), (1, 64, 64), (2, 7, 65),
              (1, 100, 255), (2, 9, 256), (1, 13, 257), (2, 37, 4095), (1, 19, 4 * 1024 + 3)]
    maxn = max(o * r * i for o, r, i in shapes) + 4
    with rd.tuning(col_waves=cw, row_waves=1, unroll=4, split=split, nontemporal=nt, path=4):
        _sweep_dim(_mask(maxn, 820 + cw + split), shapes, [0, 1, 2, 3], "cols mask", True)
        _sweep_dim(workloads.random(maxn, 821 + cw, "uniform", -30.0, 30.0), shapes, [0, 3],
                   "cols uniform", False)


def test_column_slab_plans():
    """Default plans of columns too few for one-wave tiles to reach every CU
    (one tile a block, 8 row waves joining pairs in LDS, slabs of R)."""
    import torch
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    shapes = [(1, 2000, 1000), (3, 777, 300), (1, 5000, 4095), (2, 20000, 129), (1, 300, 130),
              (4, 1031, 2048)]
    for o, r, i in shapes:
        p = rd.rd_plan_reduce(cu, o, r, i, "softmax_denom")
        assert (p.col_waves, p.row_waves, p.unroll) == (1, 8, 4), ((o, r, i), p.as_dict())
        assert p.split > 1 and p.blocks <= cu, ((o, r, i), p.as_dict())
    maxn = max(o * r * i for o, r, i in shapes) + 4
    _sweep_dim(_mask(maxn, 825), shapes, [0, 1, 3], "cols slabs mask", True)
    _sweep_dim(workloads.random(maxn, 826, "uniform", -30.0, 30.0), shapes, [0, 3],
               "cols slabs uniform", False)


SMALL = [(s, nt) for s in (1, 3) for nt in (1, 2)]


@pytest.mark.parametrize("split,nt", SMALL, ids=["s%d_nt%d" % t for t in SMALL])
def test_cols_small_kernel_shapes(split, nt):
    shapes = [(o, r, i) for i in (2, 3, 4, 5, 8, 17, 63, 64, 100, 128)
              for (o, r) in ((1, 1), (3, 7), (2, 64), (5, 130))] + [(2, 33, 129), (1, 50, 256)]
    maxn = max(o * r * i for o, r, i in shapes) + 4
    with rd.tuning(unroll=4, split=split, nontemporal=nt, path=5):
        _sweep_dim(_mask(maxn, 830 + split + nt), shapes, [0, 1, 3], "cols_small mask", True)
        _sweep_dim(workloads.random(maxn, 831 + split, "normal") * np.float32(5), shapes, [0, 3],
                   "cols_small normal*5", False)


@pytest.mark.parametrize("scale", [1e-3, 1.0, 30.0, 1000.0])
def test_random_data(scale):
    """Non-integer data of several scales, every path: m bit-exact, s within
    tolerance."""
    a = workloads.random(3_000_001, 840, "normal") * np.float32(scale)
    gm, gs = rd.rd_softmax_denom_1d(H.upload(a, 1))
    M, S = oracle.softmax_denom_dim(a, 1, a.size, 1)
    _check(gm.cpu().numpy(), gs.cpu().numpy(), M, S, "1d scale %g" % scale)
    for outer, R, inner in ((4, 1000, 4095), (300, 5000, 1), (2, 3000, 3), (64, 100, 100),
                            (1, 2_000_000, 1), (5000, 40, 1), (1, 4096, 600)):
        b = workloads.random(outer * R * inner, 841 + R, "uniform", -1.0, 1.0) * np.float32(scale)
        gm, gs = rd.rd_softmax_denom_dim(H.upload(b), outer, R, inner)
        M, S = oracle.softmax_denom_dim(b, outer, R, inner)
        _check(gm.cpu().numpy(), gs.cpu().numpy(), M, S,
               "dim scale %g %s" % (scale, (outer, R, inner)))


@pytest.mark.parametrize("step", [1e-4, 1e-2, 0.37, 5.0])
def test_rising_columns(step):
    """x_r = step * r (plus noise below step): the running maximum rises at
    nearly every term, the case where re-centring at every new maximum would
    pile up rounding; also the falling and the alternating order."""
    for outer, R, inner in ((1, 1_000_000, 1), (64, 20000, 1), (2, 5000, 300), (3, 3000, 7)):
        r = np.arange(R, dtype=np.float64)[None, :, None]
        noise = workloads.random(outer * R * inner, 850, "uniform", 0.0, 0.5).reshape(outer, R, inner)
        for name, x in (("rising", step * r + step * noise),
                        ("falling", step * (R - r) + step * noise)):
            x = x.astype(np.float32).reshape(-1)
            gm, gs = rd.rd_softmax_denom_dim(H.upload(x), outer, R, inner)
            M, S = oracle.softmax_denom_dim(x, outer, R, inner)
            _check(gm.cpu().numpy(), gs.cpu().numpy(), M, S,
                   "%s step %g %s" % (name, step, (outer, R, inner)))


def test_special_values():
    """-Inf adds nothing; all -Inf or no terms give (-Inf, 0); +Inf gives
    (+Inf, +Inf); NaN gives NaN; on every path."""
    inf, nan = np.inf, np.nan
    for outer, R, inner in ((1, 1_000_003, 1), (50, 3001, 1), (3, 999, 70), (2, 500, 4095),
                            (1, 20, 3)):
        n = outer * R * inner
        base = workloads.random(n, 860, "normal").reshape(outer, R, inner)
        cases = []
        x = base.copy(); x[0, R // 2, 0] = nan; cases.append(x)
        x = base.copy(); x[-1, R - 1, inner - 1] = inf; cases.append(x)
        x = base.copy(); x[:, :, 0] = -inf; cases.append(x)
        x = base.copy(); x[0, 0, :] = -inf; x[0, -1, :] = inf; cases.append(x)
        x = base.copy(); x[:, ::2, :] = -inf; cases.append(x)
        for k, x in enumerate(cases):
            x = x.astype(np.float32)
            gm, gs = rd.rd_softmax_denom_dim(H.upload(x.reshape(-1)), outer, R, inner)
            gm, gs = gm.cpu().numpy().reshape(-1), gs.cpu().numpy().reshape(-1)
            M, S = oracle.softmax_denom_dim(x, outer, R, inner)
            M, S = M.reshape(-1), S.reshape(-1)
            what = "special %d %s" % (k, (outer, R, inner))
            assert np.array_equal(np.isnan(gm), np.isnan(M)), what
            assert np.array_equal(np.isnan(gs), np.isnan(S)), what
            fin = ~np.isnan(M)
            H.assert_bitwise_equal_oracle(gm[fin], M[fin], what + " (max)")
            okS = ~np.isnan(S)
            assert np.array_equal(np.isinf(gs[okS]), np.isinf(S[okS])), what
            finS = okS & np.isfinite(S)
            H.assert_within_tolerance(gs[finS], S[finS], S[finS], what + " (sum)")
    e = H.upload(np.zeros(0, np.float32))
    gm, gs = rd.rd_softmax_denom_1d(e)
    assert gm.item() == -np.inf and gs.item() == 0.0
    gm, gs = rd.rd_softmax_denom_dim(e, 3, 0, 5)
    assert (gm.cpu().numpy() == -np.inf).all() and (gs.cpu().numpy() == 0.0).all()
    allneg = H.upload(np.full(70_001, -np.inf, np.float32))
    gm, gs = rd.rd_softmax_denom_1d(allneg)
    assert gm.item() == -np.inf and gs.item() == 0.0


def test_repeats_bitwise_equal():
    for k, shape in enumerate(((1, 3_000_001, 1), (300, 5000, 1), (2, 3000, 4095),
                               (64, 1000, 33), (1, 100_000, 300))):
        n = shape[0] * shape[1] * shape[2]
        x = H.upload(workloads.random(n, 870 + k, "normal") * np.float32(10))
        m0, s0 = rd.rd_softmax_denom_dim(x, *shape)
        for _ in range(4):
            m1, s1 = rd.rd_softmax_denom_dim(x, *shape)
            assert H.torch().equal(m1.view(H.torch().int32), m0.view(H.torch().int32)), shape
            assert H.torch().equal(s1.view(H.torch().int32), s0.view(H.torch().int32)), shape


def test_softmax_from_the_pair():
    """The pair gives torch's softmax and logsumexp along every dim."""
    t = H.torch()
    a = (workloads.random(6 * 70 * 8 * 9, 880, "normal") * np.float32(4)).reshape(6, 70, 8, 9)
    x = H.upload(a).view(6, 70, 8, 9)
    for dim in range(4):
        m, s = rd.softmax_denom(x, dim)
        M, S = oracle.softmax_denom_dim(a, int(np.prod(a.shape[:dim])), a.shape[dim],
                                        int(np.prod(a.shape[dim + 1:])))
        _check(m.cpu().numpy(), s.cpu().numpy(), M, S, "softmax_denom dim %d" % dim)
        sm = t.exp(x - m.unsqueeze(dim)) / s.unsqueeze(dim)
        ref = t.softmax(t.from_numpy(a.astype(np.float64)), dim).numpy()
        assert np.abs(sm.cpu().numpy() - ref).max() <= 1e-5, dim
        lse = (m + t.log(s)).cpu().numpy()
        ref = t.logsumexp(t.from_numpy(a.astype(np.float64)), dim).numpy()
        assert np.abs(lse - ref).max() <= 1e-5 * (1 + np.abs(ref).max()), dim
    m, s = rd.softmax_denom(x)
    M, S = oracle.softmax_denom_dim(a, 1, a.size, 1)
    _check(m.cpu().numpy(), s.cpu().numpy(), M, S, "softmax_denom all")


@pytest.mark.slow
@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_full_size(name):
    """The five workloads at full size, default plan: m bit-exact, s within
    tolerance on every output; 5 repeats bitwise identical."""
    w = workloads.WORKLOADS[name]
    H.say("%s softmax_denom: generating" % name)
    host = workloads.generate(w)
    if w.full_reduce:
        M, S = oracle.softmax_denom_dim(host, 1, host.size, 1)
    else:
        M, S = oracle.softmax_denom_dim(host, w.outer, w.R, w.inner)
    x = H.upload(host)
    del host

    def run():
        if w.full_reduce:
            m, s = rd.rd_softmax_denom_1d(x)
        else:
            m, s = rd.rd_softmax_denom_dim(x, w.outer, w.R, w.inner)
        return m.cpu().numpy().reshape(-1), s.cpu().numpy().reshape(-1)

    m0, s0 = run()
    _check(m0, s0, M, S, name)
    for _ in range(5):
        m1, s1 = run()
        assert np.array_equal(m1.view(np.uint32), m0.view(np.uint32))
        assert np.array_equal(s1.view(np.uint32), s0.view(np.uint32))
    del x
    H.torch().cuda.empty_cache()
