"""The C ABI from C: tests/c_abi_client.c, compiled with gcc against
include/rd.h and linked with librd.so and the oracle's liboracle.so (the
HIP runtime for device memory and a stream), runs every family of entry
points on integer data and compares with the oracle bit for bit."""
import os
import shutil
import subprocess

import pytest

import oracle
import sum_reduction_amd as rd

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_client(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    oracle.default()   # builds liboracle.so when it is missing
    libdir = os.path.dirname(rd.library_path())
    odir = os.path.dirname(oracle.LIBRARY)
    exe = str(tmp_path / "c_abi_client")
    cmd = ["gcc", "-O2", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_client.c"),
           "-o", exe, "-L" + libdir, "-lrd", "-L" + odir, "-loracle", "-L/opt/rocm/lib",
           "-lamdhip64", "-Wl,-rpath," + libdir + ":" + odir + ":/opt/rocm/lib"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "c client ok" in res.stdout
