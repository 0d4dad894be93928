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
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "librd.so")
SOURCES = ["rd_api.cpp", "rd_plan.cpp", "rd_kernels.hip", "rd_scan.hip", "rd_noalloc.hip"]
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
    return ["-O3", "-std=c++17", "--offload-arch=%s" % ARCH, "-fPIC",
            "-ffp-contract=off", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compile ``librd.so`` and ``librd_ceiling.so`` (always recompiles)."""
    _compile(SOURCES, LIBRARY, verbose)
    _compile(CEILING_SOURCES, CEILING_LIBRARY, verbose)
    return LIBRARY


def _run(cmd, verbose: bool) -> None:
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


def _compile(sources, library: str, verbose: bool) -> None:
    """Each source to an object file (in parallel: the kernel files take a
    minute or more each), then one shared library."""
    tag = "%d" % os.getpid()
    objs = [os.path.join(os.path.dirname(library),
                         "_%s.%s.o" % (os.path.splitext(s)[0], tag)) for s in sources]
    jobs = [[hipcc(), *flags(), "-c", "-o", o, os.path.join(CSRC, s)]
            for s, o in zip(sources, objs)]
    try:
        with ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as pool:
            for f in [pool.submit(_run, j, verbose) for j in jobs]:
                f.result()
        tmp = library + ".tmp%s" % tag
        _run([hipcc(), "--offload-arch=%s" % ARCH, "-shared", "-fPIC", "-o", tmp, *objs],
             verbose)
        os.replace(tmp, library)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)


if __name__ == "__main__":
    print(build(verbose=True))
