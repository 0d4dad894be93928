"""sum_reduction_amd -- fp32 sum reduction on AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``librd.so``, the HIP library whose C ABI is
``include/rd.h``.  Every step of a reduction runs in that library's kernels;
this module only checks tensors, passes their device pointers and torch's
current HIP stream, and turns status codes into exceptions.  There is no
fallback: if ``librd.so`` is missing or fails to load, every call raises.

    import torch, sum_reduction_amd as rd
    x = torch.randn(128, 4096, 4095, device="cuda")
    y = rd.rd_sum_dim(x, 128, 4096, 4095)      # [128, 4095], like x.sum(1)
    s = rd.rd_sum_1d(x)                        # 1-element tensor, x.sum()

Functions with the C names take the reduction's own sizes; ``sum`` is a
torch-style convenience (``dim=None`` or one dimension) over them.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "RdError", "RdPlan", "RdTune", "library_path", "load", "rd_sum_1d", "rd_sum_dim",
    "rd_status_string", "rd_last_hip_error", "rd_version", "rd_plan_dim",
    "rd_plan_1d", "rd_plan_reduce", "rd_tune_set", "rd_tune_supported", "sum", "tuning",
    "PATH_NAMES", "OPS", "rd_reduce_1d", "rd_reduce_dim", "reduce", "rd_cumsum_dim",
    "rd_plan_cumsum", "cumsum", "rd_cumsum_strided", "rd_plan_cumsum_strided",
    "rd_softmax_denom_1d", "rd_softmax_denom_dim", "softmax_denom", "rd_reduce_strided",
    "rd_plan_strided", "rd_softmax_denom_strided", "RD_OK", "RD_ERR_INVALID_ARG",
    "RD_ERR_NO_DEVICE", "RD_ERR_ALLOC", "RD_ERR_LAUNCH", "RD_ERR_HIP", "RD_ERR_CAPTURE",
    "RD_ERR_WORKSPACE", "RD_NOALLOC_SCRATCH_BYTES", "rd_sum_dim_noalloc",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "librd.so")

# rd_status codes (include/rd.h)
RD_OK = 0
RD_ERR_INVALID_ARG = 1
RD_ERR_NO_DEVICE = 2
RD_ERR_ALLOC = 3
RD_ERR_LAUNCH = 4
RD_ERR_HIP = 5
RD_ERR_CAPTURE = 6
RD_ERR_WORKSPACE = 7
# bytes of the fixed scratch buffer of rd_sum_dim_noalloc (include/rd.h)
RD_NOALLOC_SCRATCH_BYTES = 8 * 1024 * 1024
# rd_op: the reductions (the sum is the method; the others share its kernels)
OPS = {"sum": 0, "sumsq": 1, "max": 2, "min": 3}
# the softmax denominator's pair (maximum, shifted sum of exponentials) has
# entry points of its own; its code is accepted by rd_tune_supported
OP_SOFTMAX_DENOM = 4
PATH_NAMES = {0: "none", 1: "zero", 2: "rows", 3: "rows_short", 4: "cols",
              5: "cols_small", 6: "scan_rows", 7: "scan_cols", 8: "scan_cols_small",
              9: "strided", 10: "scan_strided"}
ORDER_NAMES = {0: "-", 1: "interleaved", 2: "blocked"}
COMBINE_NAMES = {0: "none", 1: "pass", 2: "last_block", 3: "lookback"}


class RdError(RuntimeError):
    """A non-RD_OK status from librd.so."""

    def __init__(self, status: int, where: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        super().__init__("%s: %s (hipError %d)" % (where, rd_status_string(status),
                                                    hip_error))


class RdPlan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("block_threads", ctypes.c_int32),
                ("group", ctypes.c_int32), ("col_waves", ctypes.c_int32),
                ("row_waves", ctypes.c_int32), ("unroll", ctypes.c_int32),
                ("nxcd", ctypes.c_int32), ("passes", ctypes.c_int32),
                ("combine", ctypes.c_int32),
                ("order", ctypes.c_int32), ("nontemporal", ctypes.c_int32),
                ("split", ctypes.c_int64), ("rows_per_split", ctypes.c_int64),
                ("blocks", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64)]

    def as_dict(self) -> dict:
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["path"] = PATH_NAMES.get(self.path, self.path)
        d["order"] = ORDER_NAMES.get(self.order, self.order)
        d["combine"] = COMBINE_NAMES.get(self.combine, self.combine)
        return d


class RdTune(ctypes.Structure):
    _fields_ = [("group", ctypes.c_int32), ("col_waves", ctypes.c_int32),
                ("row_waves", ctypes.c_int32), ("unroll", ctypes.c_int32),
                ("order", ctypes.c_int32), ("nontemporal", ctypes.c_int32),
                ("combine", ctypes.c_int32), ("path", ctypes.c_int32),
                ("split", ctypes.c_int64)]


_lib = None


def library_path() -> str:
    return LIBRARY


def load():
    """Load librd.so (built by ``python -m sum_reduction_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise RuntimeError("librd.so is not built (%s); run `python -m "
                           "sum_reduction_amd.build`" % LIBRARY)
    lib = ctypes.CDLL(LIBRARY)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.rd_sum_1d.argtypes = [vp, i64, vp, vp]
    lib.rd_sum_1d.restype = ctypes.c_int
    lib.rd_sum_dim.argtypes = [vp, i64, i64, i64, vp, vp]
    lib.rd_sum_dim.restype = ctypes.c_int
    lib.rd_sum_dim_noalloc.argtypes = [vp, i64, i64, i64, vp, vp]
    lib.rd_sum_dim_noalloc.restype = ctypes.c_int
    lib.rd_reduce_1d.argtypes = [vp, i64, i32, vp, vp]
    lib.rd_reduce_1d.restype = ctypes.c_int
    lib.rd_reduce_dim.argtypes = [vp, i64, i64, i64, i32, vp, vp]
    lib.rd_reduce_dim.restype = ctypes.c_int
    lib.rd_softmax_denom_1d.argtypes = [vp, i64, vp, vp, vp]
    lib.rd_softmax_denom_1d.restype = ctypes.c_int
    lib.rd_softmax_denom_dim.argtypes = [vp, i64, i64, i64, vp, vp, vp]
    lib.rd_softmax_denom_dim.restype = ctypes.c_int
    lib.rd_softmax_denom_strided.argtypes = [vp, i64, i64, i64, i64, i64, i64, vp, vp, vp]
    lib.rd_softmax_denom_strided.restype = ctypes.c_int
    lib.rd_reduce_strided.argtypes = [vp, i64, i64, i64, i64, i64, i64, i32, vp, vp]
    lib.rd_reduce_strided.restype = ctypes.c_int
    lib.rd_plan_strided.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i64,
                                    ctypes.POINTER(RdPlan)]
    lib.rd_plan_strided.restype = ctypes.c_int
    lib.rd_cumsum_dim.argtypes = [vp, i64, i64, i64, i32, vp, vp]
    lib.rd_cumsum_dim.restype = ctypes.c_int
    lib.rd_plan_cumsum.argtypes = [ctypes.c_int, i64, i64, i64, ctypes.POINTER(RdPlan)]
    lib.rd_plan_cumsum.restype = ctypes.c_int
    lib.rd_cumsum_strided.argtypes = [vp, i64, i64, i64, i64, i64, i64, i32, vp, vp]
    lib.rd_cumsum_strided.restype = ctypes.c_int
    lib.rd_plan_cumsum_strided.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i64,
                                           ctypes.POINTER(RdPlan)]
    lib.rd_plan_cumsum_strided.restype = ctypes.c_int
    lib.rd_status_string.argtypes = [ctypes.c_int]
    lib.rd_status_string.restype = ctypes.c_char_p
    lib.rd_last_hip_error.argtypes = []
    lib.rd_last_hip_error.restype = ctypes.c_int
    lib.rd_version.argtypes = []
    lib.rd_version.restype = ctypes.c_int
    lib.rd_plan_dim.argtypes = [ctypes.c_int, i64, i64, i64, ctypes.POINTER(RdPlan)]
    lib.rd_plan_dim.restype = ctypes.c_int
    lib.rd_plan_reduce.argtypes = [ctypes.c_int, i64, i64, i64, i32, ctypes.POINTER(RdPlan)]
    lib.rd_plan_reduce.restype = ctypes.c_int
    lib.rd_plan_1d.argtypes = [ctypes.c_int, i64, ctypes.POINTER(RdPlan)]
    lib.rd_plan_1d.restype = ctypes.c_int
    lib.rd_tune_set.argtypes = [ctypes.POINTER(RdTune)]
    lib.rd_tune_set.restype = ctypes.c_int
    lib.rd_tune_supported.argtypes = [i32, i32, i32, i32, i32]
    lib.rd_tune_supported.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != RD_OK:
        raise RdError(status, where, load().rd_last_hip_error())


def rd_status_string(status: int) -> str:
    return load().rd_status_string(int(status)).decode()


def rd_last_hip_error() -> int:
    return load().rd_last_hip_error()


def rd_version() -> int:
    return load().rd_version()


def rd_plan_dim(cu_count: int, outer: int, R: int, inner: int) -> RdPlan:
    plan = RdPlan()
    _check(load().rd_plan_dim(cu_count, outer, R, inner, ctypes.byref(plan)),
           "rd_plan_dim")
    return plan


def rd_plan_reduce(cu_count: int, outer: int, R: int, inner: int, op="sum") -> RdPlan:
    """Plan of rd_reduce_dim with ``op`` ("sum", "sumsq", "max", "min") or of
    rd_softmax_denom_dim (op="softmax_denom")."""
    plan = RdPlan()
    code = OP_SOFTMAX_DENOM if op == "softmax_denom" else _op_code(op)
    _check(load().rd_plan_reduce(cu_count, outer, R, inner, code, ctypes.byref(plan)),
           "rd_plan_reduce")
    return plan


def rd_plan_cumsum(cu_count: int, outer: int, R: int, inner: int) -> RdPlan:
    plan = RdPlan()
    _check(load().rd_plan_cumsum(cu_count, outer, R, inner, ctypes.byref(plan)),
           "rd_plan_cumsum")
    return plan


def rd_plan_cumsum_strided(cu_count: int, outer: int, R: int, inner: int, stride_outer: int,
                           stride_r: int, stride_inner: int) -> RdPlan:
    plan = RdPlan()
    _check(load().rd_plan_cumsum_strided(cu_count, outer, R, inner, stride_outer, stride_r,
                                         stride_inner, ctypes.byref(plan)),
           "rd_plan_cumsum_strided")
    return plan


def rd_plan_strided(cu_count: int, outer: int, R: int, inner: int, stride_outer: int,
                    stride_r: int, stride_inner: int) -> RdPlan:
    plan = RdPlan()
    _check(load().rd_plan_strided(cu_count, outer, R, inner, stride_outer, stride_r,
                                  stride_inner, ctypes.byref(plan)), "rd_plan_strided")
    return plan


def rd_plan_1d(cu_count: int, n: int) -> RdPlan:
    plan = RdPlan()
    _check(load().rd_plan_1d(cu_count, n, ctypes.byref(plan)), "rd_plan_1d")
    return plan


def rd_tune_set(tune: Optional[RdTune]):
    _check(load().rd_tune_set(ctypes.byref(tune) if tune is not None else None),
           "rd_tune_set")


def rd_tune_supported(path: str, group_or_col_waves: int, row_waves: int,
                      unroll: int, op: str = "sum") -> bool:
    code = {"rows": 2, "cols": 4, "cols_small": 5}[path]
    opc = OP_SOFTMAX_DENOM if op == "softmax_denom" else OPS[op]
    return bool(load().rd_tune_supported(opc, code, group_or_col_waves, row_waves, unroll))


class tuning:
    """Context manager that sets a process-wide tuning override, then clears it."""

    def __init__(self, **fields):
        self.tune = RdTune(**fields)

    def __enter__(self):
        rd_tune_set(self.tune)
        return self.tune

    def __exit__(self, *exc):
        rd_tune_set(None)


# --------------------------------------------------------------- tensor API
def _torch():
    import torch
    return torch


def _stream_handle(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    h = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return h or None


def _check_input(x, numel: int):
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch.Tensor")
    if x.device.type != "cuda":
        raise ValueError("x must be a GPU tensor, got device %s" % x.device)
    if x.dtype != torch.float32:
        raise ValueError("x must be float32, got %s" % x.dtype)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if x.numel() != numel:
        raise ValueError("x has %d elements, the shape needs %d" % (x.numel(), numel))


def _out_tensor(out, numel: int, device, shape):
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    if (not isinstance(out, torch.Tensor) or out.dtype != torch.float32
            or out.device != device or not out.is_contiguous() or out.numel() != numel):
        raise ValueError("out must be a contiguous float32 tensor of %d elements on %s"
                         % (numel, device))
    return out


def _op_code(op) -> int:
    if isinstance(op, str):
        if op not in OPS:
            raise ValueError("op must be one of %s" % sorted(OPS))
        return OPS[op]
    return int(op)


def rd_reduce_1d(x, op="sum", out=None, stream=None):
    """Reduction ``op`` ("sum", "sumsq", "max", "min") of all elements of the
    float32 GPU tensor ``x`` into ``out`` (a 1-element tensor, allocated when
    None).  Asynchronous on ``stream`` (default: torch's current stream)."""
    _check_input(x, x.numel() if hasattr(x, "numel") else -1)
    out = _out_tensor(out, 1, x.device, (1,))
    ptr = x.data_ptr() if x.numel() else None
    _check(load().rd_reduce_1d(ptr, x.numel(), _op_code(op), out.data_ptr(),
                               _stream_handle(stream)), "rd_reduce_1d")
    return out


def rd_reduce_dim(x, outer: int, R: int, inner: int, op="sum", out=None, stream=None):
    """out[o, i] = op over r of x[o, r, i] for x viewed as [outer, R, inner];
    ``out`` is [outer, inner] (allocated when None)."""
    _check_input(x, outer * R * inner)
    out = _out_tensor(out, outer * inner, x.device, (outer, inner))
    xp = x.data_ptr() if x.numel() else None
    optr = out.data_ptr() if out.numel() else None
    _check(load().rd_reduce_dim(xp, outer, R, inner, _op_code(op), optr,
                                _stream_handle(stream)), "rd_reduce_dim")
    return out


def _check_view(x):
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch.Tensor")
    if x.device.type != "cuda":
        raise ValueError("x must be a GPU tensor, got device %s" % x.device)
    if x.dtype != torch.float32:
        raise ValueError("x must be float32, got %s" % x.dtype)


def _check_view_span(x, outer, R, inner, stride_outer, stride_r, stride_inner):
    """The view must lie inside x's storage."""
    if min(outer, R, inner) > 0:
        if min(stride_outer, stride_r, stride_inner) < 0:
            raise ValueError("strides must be >= 0")
        last = (outer - 1) * stride_outer + (R - 1) * stride_r + (inner - 1) * stride_inner
        avail = x.untyped_storage().nbytes() // 4 - x.storage_offset()
        if last >= avail:
            raise ValueError("the view reaches float %d past x's start; its storage holds %d"
                             % (last, avail))


def rd_softmax_denom_strided(x, outer: int, R: int, inner: int, stride_outer: int,
                             stride_r: int, stride_inner: int, out_max=None, out_sum=None,
                             stream=None):
    """(m, s) of rd_softmax_denom_dim over a strided view of x's storage
    (strides in floats from x.data_ptr(); checked against the storage)."""
    _check_view(x)
    _check_view_span(x, outer, R, inner, stride_outer, stride_r, stride_inner)
    out_max = _out_tensor(out_max, outer * inner, x.device, (outer, inner))
    out_sum = _out_tensor(out_sum, outer * inner, x.device, (outer, inner))
    xp = x.data_ptr() if outer * R * inner else None
    mp = out_max.data_ptr() if out_max.numel() else None
    sp = out_sum.data_ptr() if out_sum.numel() else None
    _check(load().rd_softmax_denom_strided(xp, outer, R, inner, stride_outer, stride_r,
                                           stride_inner, mp, sp, _stream_handle(stream)),
           "rd_softmax_denom_strided")
    return out_max, out_sum


def rd_reduce_strided(x, outer: int, R: int, inner: int, stride_outer: int, stride_r: int,
                      stride_inner: int, op="sum", out=None, stream=None):
    """out[o, i] = op over r of x's storage at o*stride_outer + r*stride_r +
    i*stride_inner (floats from x.data_ptr()); ``out`` is [outer, inner].
    The view must lie inside x's storage (checked here)."""
    _check_view(x)
    _check_view_span(x, outer, R, inner, stride_outer, stride_r, stride_inner)
    out = _out_tensor(out, outer * inner, x.device, (outer, inner))
    xp = x.data_ptr() if outer * R * inner else None
    optr = out.data_ptr() if out.numel() else None
    _check(load().rd_reduce_strided(xp, outer, R, inner, stride_outer, stride_r, stride_inner,
                                    _op_code(op), optr, _stream_handle(stream)),
           "rd_reduce_strided")
    return out


def _collapse(sizes, strides):
    """(size, stride) of dims that form one strided axis, or None."""
    n, st = 1, 0
    dims = [(a, b) for a, b in zip(sizes, strides) if a != 1]
    if not dims:
        return 1, 0
    for k, (a, b) in enumerate(dims):
        if k and dims[k - 1][1] != b * a:
            return None
        n *= a
    return n, dims[-1][1]


def _view3(x, d):
    """x viewed as [outer, R, inner] with strides, reducing dim d, or None."""
    shape, strides = tuple(x.shape), tuple(x.stride())
    before = _collapse(shape[:d], strides[:d])
    after = _collapse(shape[d + 1:], strides[d + 1:])
    if before is None or after is None:
        return None
    return before[0], shape[d], after[0], before[1], strides[d], after[1]


def rd_sum_1d(x, out=None, stream=None):
    """Sum of all elements of the float32 GPU tensor ``x`` (rd_sum_1d)."""
    _check_input(x, x.numel() if hasattr(x, "numel") else -1)
    out = _out_tensor(out, 1, x.device, (1,))
    ptr = x.data_ptr() if x.numel() else None
    _check(load().rd_sum_1d(ptr, x.numel(), out.data_ptr(), _stream_handle(stream)),
           "rd_sum_1d")
    return out


def rd_sum_dim(x, outer: int, R: int, inner: int, out=None, stream=None):
    """out[o, i] = sum_r x[o, r, i] for x viewed as [outer, R, inner]; ``out``
    is [outer, inner] (allocated when None) (rd_sum_dim)."""
    _check_input(x, outer * R * inner)
    out = _out_tensor(out, outer * inner, x.device, (outer, inner))
    xp = x.data_ptr() if x.numel() else None
    optr = out.data_ptr() if out.numel() else None
    _check(load().rd_sum_dim(xp, outer, R, inner, optr, _stream_handle(stream)),
           "rd_sum_dim")
    return out


def rd_sum_dim_noalloc(x, outer: int, R: int, inner: int, out=None, stream=None):
    """rd_sum_dim without any allocation inside the library: the partial
    results of a split plan go to its fixed device scratch buffer
    (RD_NOALLOC_SCRATCH_BYTES; RdError RD_ERR_WORKSPACE when the plan needs
    more).  Calls that may overlap on one GPU share that buffer and race.
    Pass ``out`` to allocate nothing at all on the Python side either."""
    _check_input(x, outer * R * inner)
    out = _out_tensor(out, outer * inner, x.device, (outer, inner))
    xp = x.data_ptr() if x.numel() else None
    optr = out.data_ptr() if out.numel() else None
    _check(load().rd_sum_dim_noalloc(xp, outer, R, inner, optr, _stream_handle(stream)),
           "rd_sum_dim_noalloc")
    return out


def reduce(x, op="sum", dim: Optional[int] = None, out=None, stream=None):
    """torch-style reduction of a float32 GPU tensor over all elements
    (dim=None, a 0-d result; x contiguous) or over one dimension, through
    rd_reduce_1d / rd_reduce_dim, or rd_reduce_strided for a transposed,
    sliced or expanded view.  op: "sum", "sumsq", "max" or "min"."""
    if dim is None:
        return rd_reduce_1d(x, op, None if out is None else out.view(1), stream).view(())
    shape = tuple(x.shape)
    d = dim % len(shape)
    if not x.is_contiguous():
        # a strided view: reduced in place through rd_reduce_strided
        v = _view3(x, d)
        if v is None:
            raise ValueError("this view of x cannot be read as one [outer, R, inner] "
                             "strided array; make it contiguous first")
        outer, R, inner = v[:3]
        res = rd_reduce_strided(x, *v, op=op,
                                out=None if out is None else out.view(outer, inner),
                                stream=stream)
        return res.view(shape[:d] + shape[d + 1:])
    outer = 1
    for s in shape[:d]:
        outer *= s
    inner = 1
    for s in shape[d + 1:]:
        inner *= s
    res = rd_reduce_dim(x, outer, shape[d], inner, op,
                        None if out is None else out.view(outer, inner), stream)
    return res.view(shape[:d] + shape[d + 1:])


def rd_softmax_denom_dim(x, outer: int, R: int, inner: int, out_max=None, out_sum=None,
                         stream=None):
    """Softmax denominator over the middle axis of x viewed as [outer, R,
    inner]: returns (m, s), each [outer, inner] (allocated when None), with
    m = max over r and s = sum_r exp(x - c), c = m where m is finite, else 0;
    so softmax(x) = exp(x - c) / s and logsumexp(x) = c + log(s)."""
    _check_input(x, outer * R * inner)
    out_max = _out_tensor(out_max, outer * inner, x.device, (outer, inner))
    out_sum = _out_tensor(out_sum, outer * inner, x.device, (outer, inner))
    xp = x.data_ptr() if x.numel() else None
    mp = out_max.data_ptr() if out_max.numel() else None
    sp = out_sum.data_ptr() if out_sum.numel() else None
    _check(load().rd_softmax_denom_dim(xp, outer, R, inner, mp, sp, _stream_handle(stream)),
           "rd_softmax_denom_dim")
    return out_max, out_sum


def rd_softmax_denom_1d(x, out_max=None, out_sum=None, stream=None):
    """(m, s) of all elements of x: 1-element tensors (rd_softmax_denom_1d)."""
    _check_input(x, x.numel() if hasattr(x, "numel") else -1)
    out_max = _out_tensor(out_max, 1, x.device, (1,))
    out_sum = _out_tensor(out_sum, 1, x.device, (1,))
    ptr = x.data_ptr() if x.numel() else None
    _check(load().rd_softmax_denom_1d(ptr, x.numel(), out_max.data_ptr(), out_sum.data_ptr(),
                                      _stream_handle(stream)), "rd_softmax_denom_1d")
    return out_max, out_sum


def softmax_denom(x, dim: Optional[int] = None, stream=None):
    """(m, s) over all elements (dim=None, 0-d results; x contiguous) or over
    one dimension of a float32 GPU tensor (a strided view too); see
    rd_softmax_denom_dim."""
    if dim is None:
        m, s = rd_softmax_denom_1d(x, stream=stream)
        return m.view(()), s.view(())
    shape = tuple(x.shape)
    d = dim % len(shape)
    if not x.is_contiguous():
        v = _view3(x, d)
        if v is None:
            raise ValueError("this view of x cannot be read as one [outer, R, inner] "
                             "strided array; make it contiguous first")
        m, s = rd_softmax_denom_strided(x, *v, stream=stream)
        rest = shape[:d] + shape[d + 1:]
        return m.view(rest), s.view(rest)
    outer = 1
    for k in shape[:d]:
        outer *= k
    inner = 1
    for k in shape[d + 1:]:
        inner *= k
    m, s = rd_softmax_denom_dim(x, outer, shape[d], inner, stream=stream)
    rest = shape[:d] + shape[d + 1:]
    return m.view(rest), s.view(rest)


def rd_cumsum_dim(x, outer: int, R: int, inner: int, reverse: bool = True, out=None,
                  stream=None):
    """Cumulative sum along the middle axis of x viewed as [outer, R, inner]
    (reverse: from the end, y[o, r, i] = sum_{k >= r} x[o, k, i]); ``out``
    has x's shape (allocated when None; may be x itself)."""
    _check_input(x, outer * R * inner)
    out = _out_tensor(out, outer * R * inner, x.device, tuple(x.shape))
    xp = x.data_ptr() if x.numel() else None
    optr = out.data_ptr() if out.numel() else None
    _check(load().rd_cumsum_dim(xp, outer, R, inner, int(bool(reverse)), optr,
                                _stream_handle(stream)), "rd_cumsum_dim")
    return out


def rd_cumsum_strided(x, outer: int, R: int, inner: int, stride_outer: int, stride_r: int,
                      stride_inner: int, reverse: bool = True, out=None, stream=None):
    """Cumulative sum along R of the view of x's storage with element (o, r, i)
    at o*stride_outer + r*stride_r + i*stride_inner floats from x.data_ptr()
    (checked against the storage); ``out`` is the contiguous [outer, R, inner]
    result (allocated when None)."""
    _check_view(x)
    _check_view_span(x, outer, R, inner, stride_outer, stride_r, stride_inner)
    n = outer * R * inner
    out = _out_tensor(out, n, x.device, (outer, R, inner))
    xp = x.data_ptr() if n else None
    optr = out.data_ptr() if n else None
    _check(load().rd_cumsum_strided(xp, outer, R, inner, stride_outer, stride_r, stride_inner,
                                    int(bool(reverse)), optr, _stream_handle(stream)),
           "rd_cumsum_strided")
    return out


def cumsum(x, dim: int, reverse: bool = False, out=None, stream=None):
    """torch.cumsum(x, dim) (reverse=False) or torch.cumsum(x.flip(dim),
    dim).flip(dim) (reverse=True) for a float32 GPU tensor; a transposed,
    sliced or expanded view is read in place (rd_cumsum_strided), the result
    is contiguous."""
    shape = tuple(x.shape)
    d = dim % len(shape)
    if not x.is_contiguous():
        v = _view3(x, d)
        if v is None:
            raise ValueError("this view of x cannot be read as one [outer, R, inner] "
                             "strided array; make it contiguous first")
        res = rd_cumsum_strided(x, *v, reverse=reverse,
                                out=None if out is None else out.view(v[:3]), stream=stream)
        return res.view(shape)
    outer = 1
    for s in shape[:d]:
        outer *= s
    inner = 1
    for s in shape[d + 1:]:
        inner *= s
    return rd_cumsum_dim(x, outer, shape[d], inner, reverse, out, stream)


def sum(x, dim: Optional[int] = None, out=None, stream=None):
    """torch.sum(x) (x contiguous) or torch.sum(x, dim) for a float32 GPU tensor."""
    return reduce(x, "sum", dim, out, stream)
