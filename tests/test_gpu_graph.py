"""The entry points under HIP graph capture (torch.cuda.graph).

A graph records the kernels of several calls -- a split full reduce (two
kernels and a stream-ordered workspace), an axis reduce, a softmax
denominator and a split cumulative sum -- and is replayed several times with
eager work in between that changes the inputs; every replay must give the
bits of an eager call on the same inputs.  No call inside the library clears
memory with a memset node: the workspaces are written before they are read.

Skipped: the first replay of this graph once faulted (a memory aperture
violation in slab_combine_kernel, the second kernel of the [3, 50000, 70]
axis reduce, reading its graph-allocated workspace) after the plan of that
call changed; the same calls run eagerly are in bounds and pass, and the
cause was not established.  Until it is, the library refuses a call that
needs a workspace on a capturing stream (RD_ERR_CAPTURE), and these tests
stay off the GPU.
"""
import numpy as np
import pytest

import sum_reduction_amd as rd
import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _eager(xs):
    x1, x2, x3, x4 = xs
    return [rd.rd_sum_1d(x1), rd.rd_sum_dim(x2, 3, 50_000, 70),
            *rd.rd_softmax_denom_dim(x3, 2, 300_000, 1),
            rd.rd_cumsum_dim(x4, 1, 3 << 20, 1, reverse=True)]


SKIP_REASON = ("a replay of a captured workspace faulted on the GPU; cause not established, "
               "capture of workspace plans is refused (RD_ERR_CAPTURE) until it is")


@pytest.mark.skip(reason=SKIP_REASON)
def test_graph_replays_match_eager_calls():
    t = H.torch()
    rng = [workloads.random(n, 1000 + k, "normal") for k, n in
           enumerate((10_000_000, 3 * 50_000 * 70, 600_000, 3 << 20))]
    xs = [H.upload(a) for a in rng]
    outs = [t.empty(1, device="cuda"), t.empty(3, 70, device="cuda"),
            t.empty(2, 1, device="cuda"), t.empty(2, 1, device="cuda"),
            t.empty(3 << 20, device="cuda")]
    # the plans inside the graph split the work (second kernels, workspaces)
    assert rd.rd_plan_1d(256, 10_000_000).split > 1
    assert rd.rd_plan_cumsum(256, 1, 3 << 20, 1).split > 1
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):   # warm-up outside the graph, on the capture stream
        _eager(xs)
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    with t.cuda.graph(g):
        x1, x2, x3, x4 = xs
        rd.rd_sum_1d(x1, out=outs[0])
        rd.rd_sum_dim(x2, 3, 50_000, 70, out=outs[1])
        rd.rd_softmax_denom_dim(x3, 2, 300_000, 1, out_max=outs[2], out_sum=outs[3])
        rd.rd_cumsum_dim(x4, 1, 3 << 20, 1, reverse=True, out=outs[4])
    for rep in range(5):
        for x in xs:   # eager work between replays: new inputs in place
            x.mul_(1.5).add_(0.25)
        g.replay()
        t.cuda.synchronize()
        want = _eager(xs)
        t.cuda.synchronize()
        for k, (a, b) in enumerate(zip(outs, want)):
            assert t.equal(a.reshape(-1).view(t.int32), b.reshape(-1).view(t.int32)), (rep, k)
