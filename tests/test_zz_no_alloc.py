"""rd_sum_dim_noalloc through the C ABI against rd_sum_dim.

The no-allocation variant runs rd_sum_dim's plan and kernels with the
library's fixed device scratch buffer as the workspace, so its results must
be bitwise those of rd_sum_dim; both are also checked against the oracle's
tolerance.  Each case makes two no-allocation calls in a row, the second on a
smaller input, so that partial results the first left in the shared buffer
would show if the second read any of them.  Outputs sit between guard words
(nothing written outside them) and a shape whose plan needs more than the
buffer holds is refused with RD_ERR_WORKSPACE, its output untouched.
"""
import numpy as np
import pytest

import oracle
import sum_reduction_amd as rd
import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _noalloc(x, outer, R, inner, out_ptr) -> int:
    return rd.load().rd_sum_dim_noalloc(x.data_ptr() if x.numel() else None, outer, R, inner,
                                        out_ptr, H.stream_handle())


def _pair(first, second, seed, kind="normal", tune=None):
    """Two no-allocation calls (shapes first, then second) and the same two
    shapes through rd_sum_dim; bitwise equal, within the oracle's tolerance."""
    cases = []
    for k, (outer, R, inner) in enumerate((first, second)):
        a = workloads.random(outer * R * inner, seed + k, kind)
        cases.append((outer, R, inner, a, H.upload(a, k)))
    slots = H.OutSlots([o * i for o, _, i, _, _ in cases] * 2)
    ctx = rd.tuning(**tune) if tune else None
    if ctx:
        ctx.__enter__()
    try:
        for k, (outer, R, inner, _, x) in enumerate(cases):
            H.say("noalloc: %s call %d, shape %s, tune %s, workspace %d B"
                  % (("first", "second")[k], k, (outer, R, inner), tune,
                     rd.rd_plan_dim(256, outer, R, inner).workspace_bytes))
            assert _noalloc(x, outer, R, inner, slots.ptr(k)) == rd.RD_OK
        for k, (outer, R, inner, _, x) in enumerate(cases):
            assert H.call_dim(x, outer, R, inner, slots.ptr(2 + k)) == rd.RD_OK
        outs = slots.fetch()
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    for k, (outer, R, inner, a, _) in enumerate(cases):
        got, want = outs[k], outs[2 + k]
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (k, outer, R, inner)
        S, A = oracle.sum_dim(a, outer, R, inner)
        H.assert_within_tolerance(got, S, A, "noalloc %s" % ((outer, R, inner),))


def test_noalloc_full_reduce_pairs():
    # split full reduces: 1e7 floats (610 pieces of the row), then 1e6 (61)
    assert rd.rd_plan_1d(256, 10_000_000).workspace_bytes > 0
    _pair((1, 10_000_000, 1), (1, 1_000_000, 1), 300)


def test_noalloc_column_pairs():
    # split column plans: wide rows cut into slabs, then small inner sizes
    assert rd.rd_plan_dim(256, 1, 20_000, 4095).split > 1
    assert rd.rd_plan_dim(256, 3, 50_000, 70).split > 1
    _pair((1, 20_000, 4095), (1, 5_000, 4095), 310, "uniform")
    _pair((3, 50_000, 70), (2, 20_000, 70), 320)
    # narrow columns: one-wave tiles with row waves in 128 slabs, joined by a
    # wave per output (258 outputs), then a smaller such pair
    p = rd.rd_plan_dim(256, 2, 100_000, 129)
    assert (p.col_waves, p.row_waves, p.split) == (1, 8, 128), p.as_dict()
    _pair((2, 100_000, 129), (2, 30_000, 129), 330)


def test_noalloc_single_kernel_and_empty():
    # plans with no workspace, an R == 0 fill, and a row sum
    _pair((128, 256, 4095), (4, 300, 4095), 330, "uniform")
    _pair((5, 0, 7), (2, 0, 3), 340)
    _pair((4096, 2048, 1), (64, 100, 1), 350)


def test_noalloc_at_the_scratch_limit_then_refused():
    """A forced split whose partial sums nearly fill the buffer (512 slabs of
    4095 floats: 8,386,560 bytes) runs, then a smaller shape; one that needs
    more (1024 slabs) is refused with RD_ERR_WORKSPACE and writes nothing."""
    outer, R, inner = 1, 4096, 4095
    with rd.tuning(split=512):
        need = rd.rd_plan_dim(256, outer, R, inner).workspace_bytes
    assert 0.99 * rd.RD_NOALLOC_SCRATCH_BYTES < need <= rd.RD_NOALLOC_SCRATCH_BYTES
    _pair((outer, R, inner), (1, 1024, 4095), 360, "uniform", tune={"split": 512})
    with rd.tuning(split=1024):
        assert rd.rd_plan_dim(256, outer, R, inner).workspace_bytes > rd.RD_NOALLOC_SCRATCH_BYTES
        x = H.upload(workloads.random(outer * R * inner, 370, "uniform"))
        slots = H.OutSlots([inner])
        H.say("noalloc: shape %s with 1024 slabs, expecting RD_ERR_WORKSPACE" % ((outer, R, inner),))
        assert _noalloc(x, outer, R, inner, slots.ptr(0)) == rd.RD_ERR_WORKSPACE
        out = slots.fetch()[0]
    assert (out.view(np.uint32) == H.GUARD_BITS).all()


def test_noalloc_binding_and_repeat_bits():
    """The Python binding with a caller-supplied output, twice: identical bits."""
    t = H.torch()
    a = workloads.random(30_000_000, 380, "uniform")
    x = H.upload(a)
    out = t.empty(1, 1, device="cuda")
    r1 = rd.rd_sum_dim_noalloc(x, 1, a.size, 1, out=out).clone()
    r2 = rd.rd_sum_dim_noalloc(x, 1, a.size, 1, out=out).clone()
    want = rd.rd_sum_1d(x)
    assert r1.view(t.int32).item() == r2.view(t.int32).item() == want.view(t.int32).item()
