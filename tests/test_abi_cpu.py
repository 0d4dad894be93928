"""The C ABI on the host: the library loads, exports every function that
include/rd.h declares, and rejects bad arguments before any HIP call (so these
run without a GPU)."""
import ctypes
import os
import re

import pytest

import sum_reduction_amd as rd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rd.h")

OK, INVALID, NO_DEVICE = 0, 1, 2


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rd_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("rd_sum_1d", "rd_sum_dim", "rd_reduce_1d", "rd_reduce_dim",
                 "rd_status_string", "rd_last_hip_error", "rd_version", "rd_plan_dim",
                 "rd_plan_1d", "rd_tune_set", "rd_tune_supported", "rd_cumsum_dim",
                 "rd_plan_cumsum", "rd_softmax_denom_1d", "rd_softmax_denom_dim",
                 "rd_reduce_strided", "rd_plan_strided", "rd_softmax_denom_strided",
                 "rd_cumsum_strided", "rd_plan_cumsum_strided", "rd_sum_dim_noalloc"):
        assert want in names


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(rd.library_path())
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_ceiling_probes_export_their_header():
    """include/rd_ceiling.h (bandwidth probes bench.py reports as context)
    against librd_ceiling.so, and their argument checks (no GPU needed)."""
    with open(os.path.join(ROOT, "include", "rd_ceiling.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(rd_ceiling_[a-z_]+)\s*\(", text)))
    assert names == ["rd_ceiling_copy", "rd_ceiling_copy_flat", "rd_ceiling_read",
                     "rd_ceiling_read_pieces"]
    lib = ctypes.CDLL(os.path.join(ROOT, "sum_reduction_amd", "librd_ceiling.so"))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.rd_ceiling_read.argtypes = [vp, i64, i32, vp, vp]
    lib.rd_ceiling_copy.argtypes = [vp, vp, i64, i32, vp]
    buf = (ctypes.c_float * 64)()
    base = (ctypes.addressof(buf) + 15) // 16 * 16
    assert lib.rd_ceiling_read(None, 16, 1, base, None) == 1
    assert lib.rd_ceiling_read(base, 3, 1, base, None) == 1
    assert lib.rd_ceiling_read(base + 4, 16, 1, base, None) == 1     # not 16-B aligned
    assert lib.rd_ceiling_read(base, 16, 0, base, None) == 1
    lib.rd_ceiling_read_pieces.argtypes = [vp, i64, i32, vp, vp]
    assert lib.rd_ceiling_read_pieces(None, 16, 1, base, None) == 1
    assert lib.rd_ceiling_read_pieces(base + 4, 16, 1, base, None) == 1   # not 16-B aligned
    assert lib.rd_ceiling_read_pieces(base, 16, 0, base, None) == 1       # no steps
    assert lib.rd_ceiling_read_pieces(base, 16, 2000, base, None) == 1    # too many steps
    assert lib.rd_ceiling_copy(base, base + 32, 16, 1, None) == 1    # overlap
    assert lib.rd_ceiling_copy(base, None, 16, 1, None) == 1
    lib.rd_ceiling_copy_flat.argtypes = [vp, vp, i64, i32, vp]
    assert lib.rd_ceiling_copy_flat(base, base + 32, 16, 64, None) == 1   # overlap
    assert lib.rd_ceiling_copy_flat(base, base + 64, 16, 100, None) == 1  # no such workgroup
    assert lib.rd_ceiling_copy_flat(base + 4, base + 64, 16, 64, None) == 1


def test_version_and_status_strings():
    assert rd.rd_version() == 100
    names = [rd.rd_status_string(s) for s in range(8)]
    assert names == ["RD_OK", "RD_ERR_INVALID_ARG", "RD_ERR_NO_DEVICE", "RD_ERR_ALLOC",
                     "RD_ERR_LAUNCH", "RD_ERR_HIP", "RD_ERR_CAPTURE", "RD_ERR_WORKSPACE"]
    assert rd.rd_status_string(99) == "RD_ERR_UNKNOWN"
    consts = [rd.RD_OK, rd.RD_ERR_INVALID_ARG, rd.RD_ERR_NO_DEVICE, rd.RD_ERR_ALLOC,
              rd.RD_ERR_LAUNCH, rd.RD_ERR_HIP, rd.RD_ERR_CAPTURE, rd.RD_ERR_WORKSPACE]
    assert [rd.rd_status_string(c) for c in consts] == names


@pytest.fixture(scope="module")
def lib():
    return rd.load()


@pytest.fixture(scope="module")
def host_buf():
    # host memory stands in for device pointers: validation never dereferences
    buf = (ctypes.c_float * 64)()
    return ctypes.addressof(buf), buf


def test_1d_invalid_arguments(lib, host_buf):
    base, _ = host_buf
    out = base + 4 * 32
    cases = [
        (base, -1, out),            # negative n
        (base, 2 ** 62, out),       # n * 4 overflows int64
        (base, 4, None),            # null out
        (None, 4, out),             # null x with n > 0
        (base + 2, 4, out),         # x not 4-B aligned
        (base, 4, out + 1),         # out not 4-B aligned
        (base, 4, base + 8),        # out inside x
        (base, 4, base),            # out at x
    ]
    for x, n, o in cases:
        assert lib.rd_sum_1d(x, n, o, None) == INVALID, (x, n, o)


def test_dim_invalid_arguments(lib, host_buf):
    base, _ = host_buf
    out = base + 4 * 40
    cases = [
        (base, -1, 2, 2, out), (base, 2, -1, 2, out), (base, 2, 2, -1, out),
        (base, 2 ** 40, 2 ** 40, 2, out),  # size overflow
        (base, 2, 2, 2, None),             # null out, outputs exist
        (None, 2, 2, 2, out),              # null x, inputs exist
        (base + 1, 2, 2, 2, out),          # misaligned x
        (base, 2, 2, 2, out + 2),          # misaligned out
        (base, 2, 3, 4, base + 4 * 20),    # out overlaps x (x holds 24 floats)
    ]
    for x, o_, R, i, out_ in cases:
        assert lib.rd_sum_dim(x, o_, R, i, out_, None) == INVALID, (o_, R, i)
        assert lib.rd_sum_dim_noalloc(x, o_, R, i, out_, None) == INVALID, (o_, R, i)
    # nothing to write: RD_OK before any HIP call, for both
    for o_, R, i in ((0, 5, 3), (3, 5, 0), (0, 0, 0)):
        assert lib.rd_sum_dim(base, o_, R, i, out, None) == OK
        assert lib.rd_sum_dim_noalloc(base, o_, R, i, out, None) == OK


def test_noalloc_scratch_size_is_the_header_constant():
    """The binding's RD_NOALLOC_SCRATCH_BYTES is the header's, and the
    default plans of the pages' full reduces fit it (the 1D sum of 1e9
    floats has 30518 partial sums)."""
    with open(HEADER) as f:
        m = re.search(r"#define RD_NOALLOC_SCRATCH_BYTES \((\d+) \* 1024 \* 1024\)", f.read())
    assert m and int(m.group(1)) * 1024 * 1024 == rd.RD_NOALLOC_SCRATCH_BYTES
    for n in (1_000_000, 100_000_000, 1_000_000_000):
        assert 0 < rd.rd_plan_1d(256, n).workspace_bytes <= rd.RD_NOALLOC_SCRATCH_BYTES


def test_reduce_rejects_unknown_operator(lib, host_buf):
    base, _ = host_buf
    out = base + 4 * 40
    for op in (-1, 4, 5, 99):   # 4, the softmax denominator, has two outputs
        assert lib.rd_reduce_1d(base, 4, op, out, None) == INVALID
        assert lib.rd_reduce_dim(base, 2, 2, 2, op, out, None) == INVALID
    # and the other argument checks hold for every operator
    for op in range(4):
        assert lib.rd_reduce_1d(base, -1, op, out, None) == INVALID
        assert lib.rd_reduce_dim(base + 1, 2, 2, 2, op, out, None) == INVALID


def test_cumsum_invalid_arguments(lib, host_buf):
    base, _ = host_buf
    out = base + 4 * 32
    cases = [
        (base, -1, 2, 2, out), (base, 2, -1, 2, out), (base, 2, 2, -1, out),
        (base, 2 ** 40, 2 ** 40, 2, out),  # size overflow
        (base, 2, 2, 2, None),             # null out
        (None, 2, 2, 2, out),              # null x
        (base + 1, 2, 2, 2, out),          # misaligned x
        (base, 2, 2, 2, out + 2),          # misaligned out
        (base, 2, 3, 4, base + 4 * 4),     # out partly over x (x holds 24 floats)
        (base + 4 * 4, 2, 3, 4, base),     # x partly over out
    ]
    for x, o_, R, i, out_ in cases:
        for rev in (0, 1):
            assert lib.rd_cumsum_dim(x, o_, R, i, rev, out_, None) == INVALID, (o_, R, i, rev)
    # nothing to write: RD_OK, no device needed, null pointers allowed
    assert lib.rd_cumsum_dim(None, 0, 5, 3, 1, None, None) == OK
    assert lib.rd_cumsum_dim(None, 4, 0, 3, 1, None, None) == OK
    assert lib.rd_cumsum_dim(None, 4, 5, 0, 0, None, None) == OK


def test_softmax_denom_invalid_arguments(lib, host_buf):
    base, _ = host_buf
    m, s = base + 4 * 32, base + 4 * 48
    cases = [
        (base, -1, 2, 2, m, s), (base, 2, -1, 2, m, s), (base, 2, 2, -1, m, s),
        (base, 2 ** 40, 2 ** 39, 2, m, s),  # size * 8 overflows
        (base, 2, 2, 2, None, s),           # null maxima
        (base, 2, 2, 2, m, None),           # null sums
        (None, 2, 2, 2, m, s),              # null x, inputs exist
        (base + 1, 2, 2, 2, m, s),          # misaligned x
        (base, 2, 2, 2, m + 2, s),          # misaligned maxima
        (base, 2, 2, 2, m, s + 1),          # misaligned sums
        (base, 2, 3, 4, base + 4 * 20, s),  # maxima overlap x (24 floats)
        (base, 2, 3, 4, m, base),           # sums overlap x
        (base, 2, 3, 4, m, m + 4 * 7),      # sums overlap maxima (8 floats each)
        (base, 2, 3, 4, m, m),              # the same array for both
    ]
    for x, o_, R, i, mm, ss in cases:
        assert lib.rd_softmax_denom_dim(x, o_, R, i, mm, ss, None) == INVALID, (o_, R, i)
    for x, n, mm, ss in ((base, -1, m, s), (base, 2 ** 61, m, s), (base, 4, None, s),
                         (base, 4, m, None), (None, 4, m, s), (base, 4, base, s),
                         (base, 4, m, m), (base + 2, 4, m, s)):
        assert lib.rd_softmax_denom_1d(x, n, mm, ss, None) == INVALID, (n,)
    assert lib.rd_softmax_denom_dim(None, 0, 5, 3, None, None, None) == OK
    assert lib.rd_softmax_denom_dim(None, 4, 5, 0, None, None, None) == OK
    # its kernel shapes are those of the maximum
    for g, u in ((256, 16), (256, 8), (64, 8), (64, 16)):
        assert rd.rd_tune_supported("rows", g, 1, u, "softmax_denom")
    assert not rd.rd_tune_supported("rows", 256, 1, 4, "softmax_denom")
    assert rd.rd_tune_supported("cols", 8, 1, 4, "softmax_denom")
    assert not rd.rd_tune_supported("cols", 8, 2, 4, "softmax_denom")


def test_strided_invalid_arguments(lib, host_buf):
    base, _ = host_buf
    out = base + 4 * 48
    cases = [
        (base, -1, 2, 2, 4, 2, 1, out), (base, 2, 2, 2, -4, 2, 1, out),
        (base, 2, 2, 2, 4, -2, 1, out), (base, 2, 2, 2, 4, 2, -1, out),
        (base, 2, 2, 2, 2 ** 62, 2, 1, out),      # the furthest element overflows
        (base, 2, 2, 2, 4, 2, 1, None),           # null out
        (None, 2, 2, 2, 4, 2, 1, out),            # null x
        (base + 1, 2, 2, 2, 4, 2, 1, out),        # misaligned x
        (base, 2, 2, 2, 4, 2, 1, out + 2),        # misaligned out
        (base, 2, 3, 2, 20, 2, 1, base + 4 * 20), # out inside the view's span (x[0..23])
        (base, 2, 3, 2, 3, 10, 5, base + 4 * 28), # out at x[28], the furthest element (3 + 20 + 5)
    ]
    for x, o_, R, i, so, sr, si, out_ in cases:
        assert lib.rd_reduce_strided(x, o_, R, i, so, sr, si, 0, out_, None) == INVALID, (
            o_, R, i, so, sr, si)
    for op in (-1, 4, 7):
        assert lib.rd_reduce_strided(base, 2, 2, 2, 4, 2, 1, op, out, None) == INVALID
    assert lib.rd_reduce_strided(None, 0, 5, 3, 15, 3, 1, 0, None, None) == OK
    m, s2 = base + 4 * 32, base + 4 * 40
    for v in ((base, -1, 2, 2, 4, 2, 1, m, s2), (base, 2, 2, 2, 4, -2, 1, m, s2),
              (base, 2, 2, 2, 4, 2, 1, None, s2), (base, 2, 2, 2, 4, 2, 1, m, None),
              (base, 2, 2, 2, 4, 2, 1, m, m), (base, 2, 3, 2, 20, 2, 1, base + 4 * 20, s2),
              (base + 1, 2, 2, 2, 4, 2, 1, m, s2)):
        assert lib.rd_softmax_denom_strided(*v, None) == INVALID, v
    assert lib.rd_softmax_denom_strided(None, 0, 5, 3, 15, 3, 1, None, None, None) == OK
    assert lib.rd_reduce_strided(None, 4, 5, 0, 0, 0, 1, 2, None, None) == OK


def test_cumsum_strided_invalid_arguments(lib, host_buf):
    base, _ = host_buf
    out = base + 4 * 40
    cases = [
        (base, -1, 2, 2, 4, 2, 1, out), (base, 2, 2, 2, -4, 2, 1, out),
        (base, 2, 2, 2, 4, -2, 1, out), (base, 2, 2, 2, 4, 2, -1, out),
        (base, 2, 2, 2, 2 ** 62, 2, 1, out),      # the furthest element overflows
        (base, 2, 2, 2, 4, 2, 1, None),           # null out
        (None, 2, 2, 2, 4, 2, 1, out),            # null x
        (base + 1, 2, 2, 2, 4, 2, 1, out),        # misaligned x
        (base, 2, 2, 2, 4, 2, 1, out + 2),        # misaligned out
        (base, 2, 3, 2, 20, 2, 1, base + 4 * 20), # out over the view's span (x[0..23])
        (base + 4 * 8, 2, 3, 2, 6, 2, 1, base),   # the view (x[8..19]) over out[0..11]
        (base, 2, 3, 2, 1, 4, 2, base),           # in place, but not out's layout
        (base, 3, 1, 4, 8, 4, 2, base),           # in place, stride_inner 2
    ]
    for x, o_, R, i, so, sr, si, out_ in cases:
        for rev in (0, 1):
            assert lib.rd_cumsum_strided(x, o_, R, i, so, sr, si, rev, out_,
                                         None) == INVALID, (o_, R, i, so, sr, si, rev)
    # nothing to write: RD_OK, no device needed, null pointers allowed
    assert lib.rd_cumsum_strided(None, 0, 5, 3, 15, 3, 1, 1, None, None) == OK
    assert lib.rd_cumsum_strided(None, 4, 0, 3, 0, 0, 1, 0, None, None) == OK


def test_empty_output_needs_nothing(lib):
    # outer * inner == 0: nothing to write, RD_OK without a device, null ok
    assert lib.rd_sum_dim(None, 0, 5, 3, None, None) == OK
    assert lib.rd_sum_dim(None, 4, 5, 0, None, None) == OK


def _has_gpu():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="a GPU is visible")
def test_no_device_is_reported(lib, host_buf):
    base, _ = host_buf
    assert lib.rd_sum_1d(base, 8, base + 4 * 32, None) == NO_DEVICE
    assert lib.rd_sum_dim(base, 2, 2, 2, base + 4 * 32, None) == NO_DEVICE
    assert lib.rd_sum_1d(None, 0, base + 4 * 32, None) == NO_DEVICE
    assert lib.rd_cumsum_dim(base, 2, 2, 2, 1, base + 4 * 32, None) == NO_DEVICE
    assert lib.rd_cumsum_dim(base, 2, 2, 2, 1, base, None) == NO_DEVICE   # in place is valid
    assert lib.rd_softmax_denom_dim(base, 2, 2, 2, base + 4 * 32, base + 4 * 40,
                                    None) == NO_DEVICE
    assert lib.rd_softmax_denom_1d(base, 8, base + 4 * 32, base + 4 * 40, None) == NO_DEVICE
    assert lib.rd_reduce_strided(base, 2, 2, 2, 1, 4, 2, 0, base + 4 * 32, None) == NO_DEVICE
    assert lib.rd_cumsum_strided(base, 2, 2, 2, 1, 4, 2, 1, base + 4 * 32, None) == NO_DEVICE
    # in place where the view is out's layout (the strides of length-1 axes ignored)
    assert lib.rd_cumsum_strided(base, 2, 3, 4, 12, 4, 1, 0, base, None) == NO_DEVICE
    assert lib.rd_cumsum_strided(base, 1, 3, 4, 99, 4, 1, 0, base, None) == NO_DEVICE
    assert lib.rd_cumsum_strided(base, 2, 1, 4, 4, 77, 1, 0, base, None) == NO_DEVICE
    assert lib.rd_cumsum_strided(base, 2, 3, 1, 3, 1, 5, 0, base, None) == NO_DEVICE


def test_python_wrapper_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        rd.rd_sum_1d(torch.ones(4))
    with pytest.raises(ValueError):
        rd.rd_sum_dim(torch.ones(4), 1, 4, 1)
    with pytest.raises(ValueError):
        rd.rd_cumsum_dim(torch.ones(4), 1, 4, 1)
    with pytest.raises(ValueError):
        rd.rd_softmax_denom_dim(torch.ones(4), 1, 4, 1)
    with pytest.raises(ValueError):
        rd.softmax_denom(torch.ones(4))
    with pytest.raises(ValueError):
        rd.rd_cumsum_strided(torch.ones(4), 1, 4, 1, 4, 1, 1)


def test_wrapper_raises_with_status():
    with pytest.raises(rd.RdError) as e:
        rd.rd_plan_dim(0, 1, 1, 1)
    assert e.value.status == INVALID


def test_missing_library_fails_loudly(monkeypatch):
    """No silent fallback: without librd.so every entry point raises."""
    import torch
    monkeypatch.setattr(rd, "_lib", None)
    monkeypatch.setattr(rd, "LIBRARY", "/nonexistent/librd.so")
    with pytest.raises(RuntimeError, match="not built"):
        rd.load()
    with pytest.raises(RuntimeError):
        rd.rd_plan_dim(256, 1, 10, 1)
    with pytest.raises((RuntimeError, ValueError)):
        rd.rd_sum_1d(torch.ones(4))

