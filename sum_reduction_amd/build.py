"""Build ``librd.so`` (the HIP kernels and the C ABI of include/rd.h) in-tree,
and ``librd_ceiling.so`` (the bandwidth probes of include/rd_ceiling.h).

    python -m sum_reduction_amd.build          # compile for gfx950

hipcc cross-compiles for gfx950 without a GPU.  Flags:
  -O3 --offload-arch=gfx950   CDNA4 code only
  -ffp-contract=off           no fused multiply-add contraction (IEEE adds)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                              keep the compiler from emitting packed fp32 ops
  no -ffast-math              denormals and NaN/Inf semantics are kept
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "librd.so")
SOURCES = ["rd_api.cpp", "rd_plan.cpp", "rd_kernels.hip", "rd_scan.hip"]
# the bandwidth probes bench.py reports beside the reductions (include/rd_ceiling.h)
CEILING_LIBRARY = os.path.join(HERE, "librd_ceiling.so")
CEILING_SOURCES = ["rd_ceiling.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librd.so)")


def flags():
    return ["-O3", "-std=c++17", "--offload-arch=%s" % ARCH, "-fPIC", "-shared",
            "-ffp-contract=off", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compile ``librd.so`` and ``librd_ceiling.so`` (always recompiles)."""
    _compile(SOURCES, LIBRARY, verbose)
    _compile(CEILING_SOURCES, CEILING_LIBRARY, verbose)
    return LIBRARY


def _compile(sources, library: str, verbose: bool) -> None:
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = library + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *flags(), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx feature flag; that warning is noise
    noise = "is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, err))
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, library)


if __name__ == "__main__":
    print(build(verbose=True))
