"""Helpers for the GPU tests: device buffers, batched calls through the C ABI,
guard words around outputs, comparison against the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import sum_reduction_amd as rd

GUARD_BITS = np.uint32(0x7FC0DEAD)  # a quiet NaN no reduction produces
GUARD = 4                           # guard words after every output slot


def torch():
    import torch as _t
    return _t


def say(msg: str):
    """One progress line, flushed, so a run that dies names its case."""
    print(msg, file=sys.stderr, flush=True)


def upload(a: np.ndarray, offset: int = 0):
    """Device float32 tensor holding ``a`` that starts ``offset`` floats into a
    larger allocation (so its address is 4*offset bytes past a 256-B boundary)."""
    t = torch()
    a = np.ascontiguousarray(a, dtype=np.float32).reshape(-1)
    buf = t.empty(a.size + offset + 1, dtype=t.float32, device="cuda")
    view = buf[offset:offset + a.size]
    if a.size:
        view.copy_(t.from_numpy(a))
    return view


class OutSlots:
    """One device buffer cut into output slots, each followed by GUARD words
    holding GUARD_BITS; calls write to distinct slots and are checked after a
    single synchronisation."""

    def __init__(self, sizes):
        t = torch()
        self.offsets = []
        pos = GUARD
        for n in sizes:
            self.offsets.append(pos)
            pos += n + GUARD
        self.sizes = list(sizes)
        self.buf = t.empty(pos, dtype=t.int32, device="cuda")
        self.buf.fill_(int(GUARD_BITS.view(np.int32)))

    def ptr(self, k: int) -> int:
        return self.buf.data_ptr() + 4 * self.offsets[k]

    def fetch(self):
        torch().cuda.synchronize()
        host = self.buf.cpu().numpy().view(np.uint32)
        guards = np.ones(host.size, dtype=bool)
        outs = []
        for off, n in zip(self.offsets, self.sizes):
            outs.append(host[off:off + n].view(np.float32).copy())
            guards[off:off + n] = False
        bad = np.nonzero(guards & (host != GUARD_BITS))[0]
        assert bad.size == 0, "guard words overwritten at %s" % bad[:10]
        return outs


def stream_handle():
    return torch().cuda.current_stream().cuda_stream or None


def call_1d(x, out_ptr: int) -> int:
    lib = rd.load()
    return lib.rd_sum_1d(x.data_ptr() if x.numel() else None, x.numel(), out_ptr,
                         stream_handle())


def call_dim(x, outer, R, inner, out_ptr) -> int:
    lib = rd.load()
    return lib.rd_sum_dim(x.data_ptr() if x.numel() else None, outer, R, inner,
                          out_ptr, stream_handle())


def assert_bitwise_equal_oracle(got: np.ndarray, S: np.ndarray, what: str):
    """Integer-valued data: the fp32 result must equal the exact sum."""
    want = np.asarray(S, dtype=np.float64).astype(np.float32).reshape(-1)
    got = np.asarray(got, dtype=np.float32).reshape(-1)
    bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, "%s: %d mismatches, first at %d: got %r want %r" % (
        what, bad.size, bad[0], got[bad[0]], want[bad[0]])


def assert_within_tolerance(got, S, A, what: str):
    ok = oracle.within_tolerance(np.asarray(got, np.float64).reshape(-1),
                                 np.asarray(S).reshape(-1), np.asarray(A).reshape(-1))
    if not ok.all():
        k = int(np.nonzero(~ok)[0][0])
        raise AssertionError("%s: %d outputs outside 1e-5*A+1e-6, first %d: got %r "
                             "oracle %r A %r" % (what, int((~ok).sum()), k,
                                                 np.asarray(got).reshape(-1)[k],
                                                 np.asarray(S).reshape(-1)[k],
                                                 np.asarray(A).reshape(-1)[k]))
