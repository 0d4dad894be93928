"""GPU parity at full size, in the default plan (the one bench.py times).

For each of the five workloads: every output against the oracle within
|gpu - S| <= 1e-5 * A + 1e-6; 20 repeated calls bitwise identical; and the
exact invariants of fp32 summation under input scaling by 2 and negation
(both exact on every intermediate, so rd(2x) = 2 rd(x) and rd(-x) = -rd(x)).
"""
import gc
import math

import numpy as np
import pytest

import oracle
import sum_reduction_amd as rd
import workloads
from tests import gpu_helpers as H
from tests.oracle_pins import harmonic_closed_form

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

REPEATS = 20


def _run(w, x):
    if w.full_reduce:
        return rd.rd_sum_1d(x)
    return rd.rd_sum_dim(x, w.outer, w.R, w.inner)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_full_size(name):
    t = H.torch()
    w = workloads.WORKLOADS[name]
    H.say("%s: generating %d floats" % (name, w.numel))
    host = workloads.generate(w)
    H.say("%s: oracle" % name)
    if w.full_reduce:
        S, A = oracle.sum_1d(host)
        S, A = np.array([S]), np.array([A])
    else:
        S, A = oracle.sum_dim(host, w.outer, w.R, w.inner)
    H.say("%s: upload and reduce on the GPU" % name)
    x = H.upload(host)
    del host
    gc.collect()
    first = _run(w, x).cpu().numpy().reshape(-1)
    H.assert_within_tolerance(first, S, A, name)
    if name == "harmonic_1e6":
        Hn = harmonic_closed_form(w.numel)
        assert abs(float(first[0]) - Hn) <= float(oracle.tolerance(A[0])), (first, Hn)
    H.say("%s: %d repeats" % (name, REPEATS))
    outs = [_run(w, x) for _ in range(REPEATS)]
    t.cuda.synchronize()
    for k, o in enumerate(outs):
        got = o.cpu().numpy().reshape(-1)
        assert np.array_equal(got.view(np.uint32), first.view(np.uint32)), (name, k)
    del outs
    H.say("%s: invariants" % name)
    x.mul_(2.0)
    twice = _run(w, x).cpu().numpy().reshape(-1)
    assert np.array_equal(twice, 2.0 * first), name
    x.mul_(-0.5)
    neg = _run(w, x).cpu().numpy().reshape(-1)
    assert np.array_equal(neg, -first), name
    del x
    gc.collect()
    t.cuda.empty_cache()


def test_full_size_sampled_outputs_problem47():
    """Sampled outputs of the [128, 4096, 4095] reduce, each recomputed from the
    definition one at a time (oracle.sum_dim_at), including the last column
    of every outer slice (the 3-column tail lane)."""
    w = workloads.WORKLOADS["cols_128x4096x4095"]
    host = workloads.generate(w)
    got = rd.rd_sum_dim(H.upload(host), w.outer, w.R, w.inner).cpu().numpy()
    rng = np.random.default_rng(47)
    o_idx = np.concatenate([rng.integers(0, w.outer, 200), np.arange(w.outer),
                            np.arange(w.outer)])
    i_idx = np.concatenate([rng.integers(0, w.inner, 200), np.full(w.outer, w.inner - 1),
                            np.full(w.outer, w.inner - 3)])
    S, A = oracle.sum_dim_at(host, w.outer, w.R, w.inner, o_idx, i_idx)
    H.assert_within_tolerance(got[o_idx, i_idx], S, A, "problem-47 sampled")
    assert math.isfinite(float(got.sum()))
