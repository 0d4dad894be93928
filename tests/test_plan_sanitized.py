"""The planner's host code under AddressSanitizer and UBSan (CPU only).

tests/plan_fuzz.cpp and sum_reduction_amd/csrc/rd_plan.cpp are compiled with
g++ and -fsanitize=address,undefined (no GPU code is involved), then random
shapes, strides, operators and tuning requests -- including sizes near the
int64 limits -- are planned; a signed overflow, an out-of-bounds access or a
broken plan invariant fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_planner_fuzz_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "sum_reduction_amd", "csrc"),
           os.path.join(ROOT, "tests", "plan_fuzz.cpp"),
           os.path.join(ROOT, "sum_reduction_amd", "csrc", "rd_plan.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    for seed in (1, 2, 3):
        res = subprocess.run([exe, "100000", str(seed)], capture_output=True, text=True, env=env,
                             timeout=300)
        assert res.returncode == 0, res.stdout + res.stderr[-4000:]
        assert "no finding" in res.stdout
