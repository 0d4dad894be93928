"""Inputs past 2^32 elements on every path, checked against closed forms.

x repeats a pattern p of 1021 small integers (a prime length, so no axis
lines up with it): x[k] = p[k mod 1021].  Any sum of such terms has a
closed form in integers -- whole periods times sum(p) plus a partial
period -- computed here exactly in Python, with the matching sum of |x|
for the tolerance 1e-5 * A + 1e-6.  The data is built on the device from
the pattern (17-26 GB per input), so nothing that large exists on the host.
Element indices, row starts and stores all pass 2^32: a 32-bit product
anywhere in the index math shows up as a wrong output.
"""
import numpy as np
import pytest

import sum_reduction_amd as rd
import workloads
from tests import gpu_helpers as H

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

PERIOD = 1021
P = workloads.small_ints(PERIOD, 990).astype(np.int64)
PREFIX = np.concatenate([[0], np.cumsum(P)])
APREFIX = np.concatenate([[0], np.cumsum(np.abs(P))])


def F(k):
    """sum of x[0 .. k) and of |x[0 .. k)|, exactly."""
    q, r = divmod(int(k), PERIOD)
    return q * int(PREFIX[-1]) + int(PREFIX[r]), q * int(APREFIX[-1]) + int(APREFIX[r])


def column_sums(R, inner):
    """Exact sums over r < R of x[r * inner + i] for every i < inner."""
    step = inner % PERIOD
    full, rr = divmod(R, PERIOD)
    # over one full period of r the indices (step * r + i) mod PERIOD cover
    # every residue once (PERIOD is prime and step != 0)
    assert step != 0
    idx = (step * np.arange(rr, dtype=np.int64)[:, None]
           + np.arange(inner, dtype=np.int64)[None, :]) % PERIOD
    s = full * int(P.sum()) + P[idx].sum(axis=0)
    a = full * int(np.abs(P).sum()) + np.abs(P)[idx].sum(axis=0)
    return s, a


def device_input(n):
    t = H.torch()
    p = t.from_numpy(P.astype(np.float32)).cuda()
    return p.repeat(n // PERIOD + 1)[:n]


def check(got, S, A, what):
    got = np.asarray(got, np.float64).reshape(-1)
    S = np.asarray(S, np.float64).reshape(-1)
    A = np.asarray(A, np.float64).reshape(-1)
    bad = np.abs(got - S) > 1e-5 * A + 1e-6
    assert not bad.any(), "%s: %d outputs off, first %d: got %r want %r" % (
        what, bad.sum(), int(np.nonzero(bad)[0][0]), got[bad][0], S[bad][0])


def _free():
    H.torch().cuda.empty_cache()


def test_full_reduce_past_2_32():
    n = (1 << 32) + (1 << 20) + 3
    H.say("huge 1d: n=%d" % n)
    x = device_input(n)
    S, A = F(n)
    check(rd.rd_sum_1d(x).cpu().numpy(), [S], [A], "1d n=%d" % n)
    # the maximum and the softmax denominator of the same input
    assert rd.rd_reduce_1d(x, "max").item() == float(P.max())
    m, s = rd.rd_softmax_denom_1d(x)
    q, r = divmod(n, PERIOD)
    e = np.exp((P - P.max()).astype(np.float64))
    want = q * e.sum() + e[:r].sum()
    assert m.item() == float(P.max())
    assert abs(s.item() - want) <= 1e-5 * want + 1e-6, (s.item(), want)
    del x
    _free()


def test_row_sums_past_2_32():
    outer, R = 3, (1 << 31) + 7
    H.say("huge rows: [%d, %d]" % (outer, R))
    x = device_input(outer * R)
    got = rd.rd_sum_dim(x, outer, R, 1).cpu().numpy()
    S, A = [], []
    for o in range(outer):
        s1, a1 = F((o + 1) * R)
        s0, a0 = F(o * R)
        S.append(s1 - s0)
        A.append(a1 - a0)
    check(got, S, A, "rows [%d, %d]" % (outer, R))
    del x
    _free()


@pytest.mark.parametrize("R,inner", [((1 << 22) + 1, 1031), ((1 << 30) + 3, 5)])
def test_columns_past_2_32(R, inner):
    H.say("huge columns: [1, %d, %d]" % (R, inner))
    x = device_input(R * inner)
    got = rd.rd_sum_dim(x, 1, R, inner).cpu().numpy()
    S, A = column_sums(R, inner)
    check(got, S, A, "cols [1, %d, %d]" % (R, inner))
    del x
    _free()


def test_reverse_cumsum_past_2_32_in_place():
    n = (1 << 32) + 5
    H.say("huge reverse cumsum in place: n=%d" % n)
    x = device_input(n)
    rd.rd_cumsum_dim(x, 1, n, 1, reverse=True, out=x)
    tot, atot = F(n)
    ks = [0, 1, 2, n // 2, (1 << 32) - 1, 1 << 32, (1 << 32) + 1, n - 2, n - 1]
    ks += list(np.random.default_rng(991).integers(0, n, 20))
    t = H.torch()
    idx = t.tensor(ks, dtype=t.int64, device=x.device)
    got = x[idx].cpu().numpy()
    S = [tot - F(k)[0] for k in ks]
    A = [atot - F(k)[1] for k in ks]
    check(got, S, A, "reverse cumsum n=%d" % n)
    del x
    _free()
