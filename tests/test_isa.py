"""The gfx950 machine code of librd.so, read back from the library built here
(CPU only): the device code objects are taken out of the library's
.hip_fatbin section, unbundled and disassembled with the ROCm LLVM tools.

Checked: no packed-FP32 arithmetic anywhere (the library is compiled with
that feature off; with it on, hipcc -O3 turns the reduce kernels' float4
adds into some 17,000 packed instructions), and the hot loops keep the loads in flight that their
kernel shapes promise -- the 1D / row reduce 16 16-byte loads per lane, the
column reduce 4, the row scan a chunk of 8 slices, the column scan 16 rows --
issued back to back before the first wait on them, with the streaming hint.
"""
import os
import re
import shutil
import subprocess

import pytest

import sum_reduction_amd as rd

LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _tools():
    paths = [os.path.join(LLVM, t) for t in ("clang-offload-bundler", "llvm-objdump")]
    if not all(os.path.exists(p) for p in paths) or shutil.which("objcopy") is None:
        pytest.skip("needs objcopy and the ROCm LLVM tools")
    if not os.path.exists(rd.library_path()):
        pytest.skip("librd.so is not built")
    return paths


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    """{symbol: [instruction text]} for every gfx950 function in librd.so."""
    bundler, objdump = _tools()
    tmp = tmp_path_factory.mktemp("isa")
    # work on a copy: objcopy rewrites its input file unless given an output
    # file, and this process has the library mapped
    lib, fat = str(tmp / "librd.so"), str(tmp / "fatbin")
    shutil.copyfile(rd.library_path(), lib)
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", lib, fat],
                   check=True, capture_output=True)
    data = open(fat, "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)] + [len(data)]
    assert len(starts) >= 2, "no offload bundle in .hip_fatbin"
    funcs = {}
    for k in range(len(starts) - 1):  # one bundle per translation unit
        b, co = str(tmp / ("b%d" % k)), str(tmp / ("co%d.o" % k))
        open(b, "wb").write(data[starts[k]:starts[k + 1]])
        subprocess.run([bundler, "--unbundle", "--type=o", "--targets=" + TARGET,
                        "--input=" + b, "--output=" + co], check=True, capture_output=True)
        dis = subprocess.run([objdump, "-d", "--mcpu=gfx950", co], check=True,
                             capture_output=True, text=True).stdout
        cur = None
        for line in dis.splitlines():
            m = re.match(r"^[0-9a-f]+ <(.*)>:$", line)
            if m:
                cur = m.group(1)
                funcs[cur] = []
            elif cur and line.strip():
                funcs[cur].append(line.split("//")[0].strip())
    return funcs


def _one(kernels, *parts):
    names = [n for n in kernels if all(p in n for p in parts)]
    assert len(names) == 1, (parts, names)
    return kernels[names[0]]


def _load_runs(body):
    """Global loads issued back to back before each wait on vector memory."""
    runs, cur = [], []
    for ins in body:
        op = ins.split()[0] if ins else ""
        if op.startswith("global_load"):
            cur.append(ins)
        elif op == "s_waitcnt" and "vmcnt" in ins:
            runs.append(cur)
            cur = []
    return runs


def test_the_library_has_the_kernels(kernels):
    for part in ("rows_kernel", "cols_kernel", "cols_small_kernel", "rows_short_tile_kernel",
                 "strided_kernel", "scan_rows_kernel", "scan_rows_block_kernel",
                 "scan_rows_stream_kernel",
                 "scan_cols_kernel", "scan_small_kernel",
                 "scan_tile_out_kernel", "scan_tile_in_kernel", "scan_strided_kernel"):
        assert any(part in n for n in kernels), part


def test_no_packed_fp32_arithmetic(kernels):
    bad = {"v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32"}
    found = [(n, i) for n, body in kernels.items() for i in body if i.split()[:1] and
             i.split()[0] in bad]
    assert not found, found[:5]


@pytest.mark.parametrize("parts,loads", [
    (("rows_kernelILi0ELi256ELi16ELb1E",), 16),          # 1D / row sum, U = 16
    (("cols_kernelILi0ELi8ELi1ELi4ELb1E",), 4),          # column sum, U = 4
    (("scan_rows_block_kernelILb1ELi8ELi8ELb1E",), 8),   # reverse row scan, 8 waves x 8 slices
    (("scan_rows_block_kernelILb1ELi16ELi8ELb1E",), 8),  # the same, 16 waves
    (("scan_cols_kernelILb1ELi4ELi16ELi8ELb1E",), 16),   # column scan, 16 rows
], ids=["rows_sum", "cols_sum", "scan_rows", "scan_rows_wide", "scan_cols"])
def test_hot_loops_keep_their_loads_in_flight(kernels, parts, loads):
    # per run: the 16-byte loads with the streaming hint
    streamed = [sum(1 for i in r if i.split()[0] == "global_load_dwordx4" and
                    re.search(r"\bnt\b", i)) for r in _load_runs(_one(kernels, *parts))]
    assert max(streamed) >= loads, streamed
