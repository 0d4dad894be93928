"""The entry points under HIP graph capture (torch.cuda.graph).

Run: a call whose plan needs a workspace is refused on a capturing stream
(RD_ERR_CAPTURE) and records nothing; calls whose plan is one kernel with no
workspace are captured and replayed several times, with eager work in
between that changes the inputs, and every replay gives the bits of an
eager call on the same inputs.

Skipped: a graph of calls with workspaces (a split full reduce -- two
kernels and a stream-ordered workspace --, a split axis reduce, a softmax
denominator, a split cumulative sum).  Its first replay once faulted (a
memory aperture violation in slab_combine_kernel, the second kernel of the
[3, 50000, 70] axis reduce, reading its graph-allocated workspace) after the
plan of that call changed; the same calls run eagerly are in bounds and
pass, and the cause was not established.  Until it is, the library refuses
such calls while capturing, and that test stays off the GPU.
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


def test_capture_refuses_workspace_plans():
    """A call whose plan needs a workspace returns RD_ERR_CAPTURE while its
    stream is being captured, and records nothing; the capture goes on."""
    t = H.torch()
    x = H.upload(workloads.random(1_000_000, 2001, "normal"))
    y = t.zeros(16, device="cuda")
    assert rd.rd_plan_1d(256, 1_000_000).workspace_bytes > 0
    rd.rd_sum_1d(x)  # the device's set-up happens outside the capture
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    statuses = []
    with t.cuda.graph(g):
        try:
            rd.rd_sum_1d(x)
        except rd.RdError as e:
            statuses.append(e.status)
        y.add_(1.0)
    assert statuses == [rd.RD_ERR_CAPTURE]
    for _ in range(3):
        g.replay()
    t.cuda.synchronize()
    assert float(y.sum()) == 3.0 * 16


def test_large_row_scan_captures_as_one_kernel():
    """A row scan whose plan is the look-back kernel with one piece per row
    (an array of 1 GiB) needs a workspace only for its ticket: on a
    capturing stream the workgroup-per-row kernel with the same chunk runs
    instead, and its replays give the eager call's bits."""
    t = H.torch()
    o, r = 8192, 32768
    p = rd.rd_plan_cumsum(256, o, r, 1)
    assert p.as_dict()["combine"] == "lookback" and p.split == 1
    x = H.upload(workloads.random(o * r, 2002, "normal"))
    out = t.empty(o * r, device="cuda")
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        rd.rd_cumsum_dim(x, o, r, 1, reverse=True, out=out)   # set-up outside the capture
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        rd.rd_cumsum_dim(x, o, r, 1, reverse=True, out=out)
    for rep in range(3):
        x.mul_(1.5).add_(0.25)
        g.replay()
        t.cuda.synchronize()
        want = rd.rd_cumsum_dim(x, o, r, 1, reverse=True)   # eager: the look-back kernel
        t.cuda.synchronize()
        assert t.equal(out.view(t.int32), want.view(t.int32)), rep


def test_single_kernel_plans_replay():
    """Calls whose plan is one kernel and no workspace (a column reduce, a row
    reduce with a workgroup per row, a cumulative sum of uncut rows) capture
    and replay: every replay, with eager work changing the inputs in between,
    gives the bits of an eager call."""
    t = H.torch()
    shapes = [(128, 256, 4095), (4096, 2048, 1)]
    for o, r, i in shapes:
        p = rd.rd_plan_dim(256, o, r, i)
        assert p.split == 1 and p.workspace_bytes == 0, (o, r, i)
    assert rd.rd_plan_cumsum(256, 2048, 5000, 1).workspace_bytes == 0
    xs = [H.upload(workloads.random(o * r * i, 2100 + k, "normal"))
          for k, (o, r, i) in enumerate(shapes)]
    xc = H.upload(workloads.random(2048 * 5000, 2110, "normal"))
    outs = [t.empty(o * i, device="cuda") for o, r, i in shapes]
    oc = t.empty(2048 * 5000, device="cuda")
    for (o, r, i), x, out in zip(shapes, xs, outs):  # warm-up outside the capture
        rd.rd_sum_dim(x, o, r, i, out=out)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        for (o, r, i), x, out in zip(shapes, xs, outs):
            rd.rd_sum_dim(x, o, r, i, out=out)
        rd.rd_cumsum_dim(xc, 2048, 5000, 1, reverse=True, out=oc)
    for rep in range(4):
        for x in xs + [xc]:
            x.mul_(1.25).add_(0.5)
        g.replay()
        t.cuda.synchronize()
        for (o, r, i), x, out in zip(shapes, xs, outs):
            want = rd.rd_sum_dim(x, o, r, i)
            assert t.equal(out.view(t.int32), want.reshape(-1).view(t.int32)), (rep, o, r, i)
        want = rd.rd_cumsum_dim(xc, 2048, 5000, 1, reverse=True)
        assert t.equal(oc.view(t.int32), want.reshape(-1).view(t.int32)), (rep, "cumsum")


_FIRST_CALL = r"""
import sys
sys.path.insert(0, sys.argv[1])
import torch
import sum_reduction_amd as rd
x = torch.ones(128 * 256 * 4095, device="cuda")
y = torch.zeros(16, device="cuda")
y.add_(0.0)                      # torch's own set-up, outside the capture
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
st = []
with torch.cuda.graph(g):
    try:
        rd.rd_sum_dim(x, 128, 256, 4095)   # the library's first call on the device
    except rd.RdError as e:
        st.append(e.status)
    y.add_(1.0)
g.replay()
torch.cuda.synchronize()
assert st == [rd.RD_ERR_CAPTURE], st
assert float(y.sum()) == 16.0
out = rd.rd_sum_dim(x, 128, 256, 4095)     # set up now, outside the capture
assert float(out.min()) == 256.0 and float(out.max()) == 256.0
print("first-call-ok")
"""


def test_first_call_under_capture_is_refused():
    """The library's first call on a device sets the device up (it allocates
    and synchronizes); on a capturing stream it returns RD_ERR_CAPTURE before
    any of that, and the capture stays valid.  Needs a process whose library
    has not been used yet: one child process."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, "-c", _FIRST_CALL, root], capture_output=True,
                         text=True, timeout=240)
    assert res.returncode == 0 and "first-call-ok" in res.stdout, res.stdout + res.stderr[-3000:]
