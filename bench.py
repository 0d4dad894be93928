"""Benchmark of the fp32 sum reduction on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME ...]

One step is one pass of the whole reduction path over the two workloads the
headline metric is quoted on:

    rd_sum_1d  over normal_1e9          (1e9 floats, N(0,1), 4.0 GB)
    rd_sum_dim over cols_128x4096x4095  ([128, 4096, 4095] reduced over dim 1,
                                         U[0,1), 8.59 GB)

Inputs are generated on the host (workloads.py), copied to HBM before the
timed region, and stay resident.  W untimed steps, then K timed steps between
two synchronisations.  `value` is the step's algorithmic bytes (every input
read once, every output written once) over the step time, in GB/s.  Each call
is also bracketed by HIP events on the stream the library launches on, which
gives the per-call times of the `per_workload` block and the average launch
time of the dominant kernel for `roofline`.

`cpu_baseline` times the oracle (oracle/, fp64, the test reference) on the
host over the same workloads: the full reduce single-threaded (it is one
sequential loop), the axis reduce over all host threads.  The GPU results of
the last step are checked against those oracle results (`parity`).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HBM GB/s & % of peak: fp32 sum n=1e9; [128,4096,4095] dim-1 reduce"
PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
STEP_WORKLOADS = ["normal_1e9", "cols_128x4096x4095"]
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "sum_reduction_amd", "csrc")
# the device code of the reductions and of the scans (a counter summary taken
# on other sources no longer describes the kernels)
KERNEL_SOURCES = {"reduce": ("rd_kernels.hip", "rd_device.h"),
                  "scan": ("rd_scan.hip", "rd_device.h")}


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_digest(kind: str = "reduce") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kind: str = "reduce"):
    """HBM bytes per launch of the workload's main kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source
    (else None)."""
    path = os.path.join(PROFILES, "traffic_%s.md" % workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    digest = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    value = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not digest or not value or digest.group(1) != kernel_source_digest(kind):
        return None
    return float(value.group(1))


def kernel_name(plan: dict) -> str:
    """The main-pass kernel a plan launches, as the profiler names it."""
    nt = "true" if plan["nontemporal"] else "false"
    if plan["path"] == "cols":  # first template argument: the operator (0 = sum)
        return "cols_kernel<0, %d, %d, %d, %s>" % (plan["col_waves"], plan["row_waves"],
                                                   plan["unroll"], nt)
    if plan["path"] == "rows":
        return "rows_kernel<0, %d, %d, %s>" % (plan["group"], plan["unroll"], nt)
    return plan["path"] + "_kernel"


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", action="append", default=None,
                    help="bench these workloads instead of the default step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--report", action="store_true",
                    help="instead of the step line: one JSON line per workload (all five "
                         "unless --workload is given), warm and cold GPU times, the oracle's "
                         "CPU time and the parity check")
    ap.add_argument("--dim-shape", action="append", default=None, metavar="OxRxI",
                    help="with --report: also an axis reduce of this [outer, R, inner] "
                         "shape, U[0,1) data from seed 0")
    ap.add_argument("--op", action="append", default=None,
                    choices=["sum", "sumsq", "max", "min", "softmax_denom"],
                    help="with --report: the reductions to time (default: sum); "
                    "softmax_denom writes the pair (max, shifted sum of exp)")
    ap.add_argument("--strided", action="store_true",
                    help="with --report: sums, then cumulative sums, over strided views of "
                    "a [32768, 32768] array (transposed, every other row, every third "
                    "column) instead")
    ap.add_argument("--scan", action="store_true",
                    help="with --report: the cumulative sums instead (problem 91's "
                    "[32768, 32768] rows, then each --scan-shape)")
    ap.add_argument("--scan-shape", action="append", default=None, metavar="OxRxI",
                    help="with --report --scan: also a cumulative sum of this shape")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the trivial read / copy kernels timed after the step")
    ap.add_argument("--reps", type=int, default=0,
                    help="with --report: timed calls per measurement (default 200 "
                    "under 1 GiB, else 30)")
    ap.add_argument("--no-oracle", action="store_true",
                    help="with --report: skip the oracle and the parity check "
                    "(short runs under a profiler)")
    ap.add_argument("--copy-probe-bytes", type=int, default=0,
                    help="only run a device-to-device copy of this many bytes 3 times "
                         "(a known-size kernel for calibrating HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: there is no multi-GPU path here "
              "(a multi-GPU reduce would split the input and gather one partial "
              "per GPU; it is not built)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import sum_reduction_amd as rd
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    rd.load()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda", 0)
    if args.copy_probe_bytes:
        n = args.copy_probe_bytes // 4
        src = torch.zeros(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": 4 * n, "copies": 3}), flush=True)
        return 0
    props = torch.cuda.get_device_properties(dev)
    cu = props.multi_processor_count
    if args.report:
        if args.strided:
            return report_strided(args, dev, cu)
        return report_scan(args, dev, cu) if args.scan else report(args, dev, cu)
    names = args.workload or STEP_WORKLOADS
    ws = [workloads.WORKLOADS[n] for n in names]

    host, xs = {}, {}
    for w in ws:
        log("generating %s (%d floats)" % (w.name, w.numel))
        host[w.name] = workloads.generate(w)
        xs[w.name] = torch.from_numpy(host[w.name]).to(dev)
    outs = {w.name: torch.empty(w.out_numel, dtype=torch.float32, device=dev) for w in ws}
    plans = {w.name: (rd.rd_plan_1d(cu, w.numel) if w.full_reduce
                      else rd.rd_plan_dim(cu, w.outer, w.R, w.inner)).as_dict()
             for w in ws}
    torch.cuda.synchronize()

    def one_step(events=None):
        for k, w in enumerate(ws):
            if events is not None:
                events[k][0].record()
            if w.full_reduce:
                rd.rd_sum_1d(xs[w.name], out=outs[w.name])
            else:
                rd.rd_sum_dim(xs[w.name], w.outer, w.R, w.inner, out=outs[w.name])
            if events is not None:
                events[k][1].record()

    log("warmup %d steps" % args.warmup)
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in ws] for _ in range(K)]
    log("timing %d steps" % K)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        one_step(ev[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    step_bytes = sum(w.algorithmic_bytes for w in ws)
    value = step_bytes * K / elapsed / 1e9
    per = {}
    for k, w in enumerate(ws):
        ms = sorted(ev[s][k][0].elapsed_time(ev[s][k][1]) for s in range(K))
        med, mean = ms[len(ms) // 2], sum(ms) / len(ms)
        per[w.name] = {
            "ms_median": round(med, 5), "ms_mean": round(mean, 5),
            "ms_min": round(ms[0], 5), "ms_max": round(ms[-1], 5),
            "GBps_median": round(w.algorithmic_bytes / med / 1e6, 1),
            "frac_of_peak": round(w.algorithmic_bytes / med / 1e6 / PEAK_GBS, 4),
            "algorithmic_bytes": w.algorithmic_bytes,
            "plan": plans[w.name],
        }

    # dominant kernel: the workload whose call takes longest; its call is one
    # kernel launch when its plan has a single pass
    dom = max(per, key=lambda n: per[n]["ms_mean"])
    dw = workloads.WORKLOADS[dom]
    achieved = dw.algorithmic_bytes / (per[dom]["ms_mean"] * 1e-3) / 1e9
    traffic = measured_traffic(dom)
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic,
        "kernel": kernel_name(plans[dom]),
        "workload": dom, "launches_per_call": plans[dom]["passes"],
        "kernel_source_sha256_16": kernel_source_digest(),
    }

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / K, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": " + ".join(names),
                   "shapes": {w.name: list(w.shape) for w in ws},
                   "step_bytes": step_bytes,
                   "frac_of_peak": round(value / PEAK_GBS, 4)},
        "roofline": roofline,
        "per_workload": per,
        "device": {"name": props.name, "cu": cu, "gcn_arch": getattr(props, "gcnArchName", "")},
    }

    if not args.no_ceiling:
        src = max(xs.values(), key=lambda t: t.numel())
        log("ceiling probes on %d floats" % src.numel())
        result["ceiling"] = measure_ceiling(src, achieved)

    if not args.no_cpu_baseline:
        import oracle

        threads = oracle.default_threads()
        log("cpu baseline: oracle on the host (axis reduce over %d threads)" % threads)
        results, parity = {}, True
        legs = {w.name: [] for w in ws}
        reps = 0
        # each leg timed on its own, the whole step repeated until ~5 s of CPU
        # work (at most 5 times); median per leg
        while reps < 5 and sum(sum(v) for v in legs.values()) < 5.0:
            for w in ws:
                t0 = time.perf_counter()
                if w.full_reduce:
                    S, A = oracle.sum_1d(host[w.name])
                    S, A = np.array([S]), np.array([A])
                else:
                    S, A = oracle.sum_dim(host[w.name], w.outer, w.R, w.inner, threads)
                legs[w.name].append(time.perf_counter() - t0)
                if reps == 0:
                    got = outs[w.name].cpu().numpy()
                    ok = bool(oracle.within_tolerance(got.reshape(-1), S.reshape(-1),
                                                      A.reshape(-1)).all())
                    parity &= ok
                    results[w.name] = ok
            reps += 1
        leg_info = {}
        step_s = 0.0
        for w in ws:
            med = sorted(legs[w.name])[len(legs[w.name]) // 2]
            step_s += med
            # the full reduce is one sequential loop in index order; the axis
            # reduce runs independent outputs on every host thread
            leg_info[w.name] = {"s_median": round(med, 4),
                                "GBps": round(w.algorithmic_bytes / med / 1e9, 3),
                                "threads": 1 if w.full_reduce else threads}
        result["cpu_baseline"] = {
            "value": round(step_bytes / step_s / 1e9, 3), "unit": "GB/s",
            "cores": max(v["threads"] for v in leg_info.values()), "kind": "oracle",
            "legs": leg_info,
            "sample": "the whole step, each leg timed on its own (median of %d runs): the full "
                      "reduce on 1 thread (the oracle's loop is sequential), the axis reduce "
                      "over %d threads; value = step bytes / sum of the leg medians "
                      "(%.3f s); %s" % (reps, threads, step_s, cpu_model()),
        }
        result["parity"] = {"ok": parity, "per_workload": results,
                            "rule": "|gpu - S| <= 1e-5*sum|x| + 1e-6 per output"}

    print(json.dumps(result), flush=True)
    return 0


def measure_ceiling(src, achieved_gbs):
    """Bandwidth of trivial kernels on this GPU (librd_ceiling.so): reads of
    `src` -- grid-stride over a few grid sizes, and pieces of a few lengths,
    one per workgroup, 16 loads in flight per lane -- and a copy of it,
    grid-stride or one 16-byte chunk per thread over a few workgroup sizes;
    best median of 10 event-timed launches.  The best read is the achievable
    read rate the dominant kernel is compared with; the roofline fraction
    stays relative to the published 8 TB/s."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "sum_reduction_amd", "librd_ceiling.so"))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.rd_ceiling_read.argtypes = [vp, i64, i32, vp, vp]
    lib.rd_ceiling_read_pieces.argtypes = [vp, i64, i32, vp, vp]
    lib.rd_ceiling_copy.argtypes = [vp, vp, i64, i32, vp]
    lib.rd_ceiling_copy_flat.argtypes = [vp, vp, i64, i32, vp]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream or None
    n = src.numel() // 4 * 4
    # one float per grid-stride thread (at most 8192 x 256) or per piece
    # (at most ceil(n/4 / 4096))
    sink = torch.empty(max((1 << 13) * 256, n // 4 // 4096 + 1), dtype=torch.float32,
                       device=src.device)
    dst = torch.empty(n, dtype=torch.float32, device=src.device)

    def best(fn, grids, nbytes):
        out = (0.0, 0)
        for g in grids:
            assert fn(g) == 0
            torch.cuda.synchronize()
            ms = []
            for _ in range(10):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn(g)
                b.record(stream)
                b.synchronize()
                ms.append(a.elapsed_time(b))
            gbs = nbytes / sorted(ms)[len(ms) // 2] / 1e6
            out = max(out, (gbs, g))
        return out

    rd_gbs, rd_g = best(lambda g: lib.rd_ceiling_read(src.data_ptr(), n, g, sink.data_ptr(), sh),
                        (256, 512, 1024, 2048, 4096, 8192), 4 * n)
    pc_gbs, pc_s = best(lambda s: lib.rd_ceiling_read_pieces(src.data_ptr(), n, s,
                                                             sink.data_ptr(), sh),
                        (1, 2, 4, 8), 4 * n)
    cp_gbs, cp_g = best(lambda g: lib.rd_ceiling_copy(src.data_ptr(), dst.data_ptr(), n, g, sh),
                        (2048, 8192, 32768), 8 * n)
    fl_gbs, fl_t = best(lambda t: lib.rd_ceiling_copy_flat(src.data_ptr(), dst.data_ptr(), n, t,
                                                           sh),
                        (64, 256, 1024), 8 * n)
    del dst, sink
    torch.cuda.empty_cache()
    copy_shape = ("grid-stride, %d workgroups of 256" % cp_g if cp_gbs >= fl_gbs else
                  "one 16-byte chunk per thread, workgroups of %d" % fl_t)
    read = max(rd_gbs, pc_gbs)
    read_shape = ("grid-stride, %d workgroups of 256" % rd_g if rd_gbs >= pc_gbs else
                  "a piece of %d KB per workgroup of 256, 16 loads in flight per lane"
                  % (pc_s * 64))
    return {"read_GBps": round(read, 1), "read_shape": read_shape,
            "read_grid_stride_GBps": round(rd_gbs, 1), "read_pieces_GBps": round(pc_gbs, 1),
            "copy_GBps": round(max(cp_gbs, fl_gbs), 1), "copy_shape": copy_shape,
            "copy_grid_stride_GBps": round(cp_gbs, 1), "bytes_read": 4 * n,
            "roofline_achieved_over_read": round(achieved_gbs / read, 4),
            "kind": "trivial kernels, 16-byte nontemporal accesses (include/rd_ceiling.h)"}


# Context figures printed by the pages for the same operation (another machine):
# "High-Performance Reduction Kernels" README, results on an NVIDIA T4 (sm_75),
# fastest implementation per n, averaged over 100 launches.
PAGES_T4 = {
    "harmonic_1e6": {"ms": 0.0137, "impl": "CUDA C", "hardware": "NVIDIA T4"},
    "uniform_1e8": {"ms": 1.4716, "impl": "CUDA C", "hardware": "NVIDIA T4"},
    "normal_1e9": {"ms": 14.4983, "impl": "PyTorch", "hardware": "NVIDIA T4"},
}


def report(args, dev, cu):
    """One JSON line per workload: GPU time warm (back to back) and cold (a
    1 GiB write between calls evicts the caches, outside the timed events),
    GB/s and fraction of 8 TB/s, the oracle's CPU time, and parity."""
    import numpy as np
    import torch

    import oracle
    import sum_reduction_amd as rd
    import workloads

    threads = oracle.default_threads()
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    todo = [workloads.WORKLOADS[n] for n in (args.workload or
                                             ([] if args.dim_shape else list(workloads.WORKLOADS)))]
    for spec in args.dim_shape or []:
        o, r, i = (int(v) for v in spec.lower().split("x"))
        todo.append(workloads.Workload("shape_%dx%dx%d" % (o, r, i), (o, r, i), o, r, i,
                                       "uniform", seed=0))
    for w in todo:
        host = workloads.generate(w)
        x = torch.from_numpy(host).to(dev)
        out = torch.empty(2 * w.out_numel, dtype=torch.float32, device=dev)
        for op in (args.op or ["sum"]):
            log("report: %s %s" % (w.name, op))
            print(json.dumps(report_one(w, op, host, x, out, flush, threads, cu, args)),
                  flush=True)
        del x, out, host
        torch.cuda.empty_cache()
    return 0


# Strided views of one [N, N] float array, N = 32768 (4.3 GB), seed 3 normal
# data: (name, outer, R, inner, stride_outer, stride_r, stride_inner), the
# torch expression it stands for, and the bytes the view holds.
STRIDED_N = 32768
STRIDED_VIEWS = [
    ("rows_of_transpose", STRIDED_N, STRIDED_N, 1, 1, STRIDED_N, 1, "x.t().sum(1)"),
    ("cols_of_transpose", 1, STRIDED_N, STRIDED_N, 0, 1, STRIDED_N, "x.t().sum(0)"),
    ("every_other_row", 1, STRIDED_N // 2, STRIDED_N, 0, 2 * STRIDED_N, 1, "x[::2].sum(0)"),
    ("row_halves", STRIDED_N, STRIDED_N // 2, 1, STRIDED_N, 1, 1, "x[:, :N/2].sum(1)"),
    ("every_third_column", 1, STRIDED_N // 8, STRIDED_N // 3, 0, 8 * STRIDED_N, 3,
     "x[::8, ::3].sum(0)"),
]


# the same views scanned (rd_cumsum_strided, forward): the output is the
# contiguous array of the view's shape
STRIDED_SCAN_VIEWS = [
    ("rows_of_transpose", STRIDED_N, STRIDED_N, 1, 1, STRIDED_N, 1, "x.t().cumsum(1)"),
    ("cols_of_transpose", 1, STRIDED_N, STRIDED_N, 0, 1, STRIDED_N, "x.t().cumsum(0)"),
    ("every_other_row", 1, STRIDED_N // 2, STRIDED_N, 0, 2 * STRIDED_N, 1, "x[::2].cumsum(0)"),
    ("row_halves", STRIDED_N, STRIDED_N // 2, 1, STRIDED_N, 1, 1, "x[:, :N/2].cumsum(1)"),
    ("every_third_column", 1, STRIDED_N // 8, STRIDED_N // 3, 0, 8 * STRIDED_N, 3,
     "x[::8, ::3].cumsum(0)"),
]


def report_strided(args, dev, cu):
    """One JSON line per strided view: GPU time warm, GB/s over the bytes the
    view holds, its plan, parity against the oracle on a contiguous copy."""
    import numpy as np
    import torch

    import oracle
    import sum_reduction_amd as rd
    import workloads

    threads = oracle.default_threads()
    n = STRIDED_N
    host = workloads.random(n * n, 3, "normal")
    x = torch.from_numpy(host).to(dev)
    for name, o, R, i, so, sr, si, expr in STRIDED_VIEWS:
        log("report: strided %s" % name)
        out = torch.empty(o * i, dtype=torch.float32, device=dev)

        def call():
            rd.rd_reduce_strided(x, o, R, i, so, sr, si, "sum", out=out)

        reps = args.reps or 30
        ms = _median_ms(call, reps)
        nbytes = 4 * (o * R * i + o * i)
        plan = rd.rd_plan_strided(cu, o, R, i, so, sr, si).as_dict()
        line = {"view": name, "torch": expr, "shape": [o, R, i], "strides": [so, sr, si],
                "view_bytes": nbytes, "ms_median": round(ms, 5),
                "GBps": round(nbytes / ms / 1e6, 1),
                "frac_of_peak": round(nbytes / ms / 1e6 / PEAK_GBS, 4),
                "plan": plan, "reps": reps}
        if not args.no_oracle:
            v = np.lib.stride_tricks.as_strided(host, shape=(o, R, i),
                                                strides=(4 * so, 4 * sr, 4 * si),
                                                writeable=False)
            S, A = oracle.sum_dim(np.ascontiguousarray(v), o, R, i, threads)
            got = out.cpu().numpy().reshape(-1)
            line["parity"] = {"ok": bool(oracle.within_tolerance(got, S.reshape(-1),
                                                                 A.reshape(-1)).all())}
        print(json.dumps(line), flush=True)
        del out
    for name, o, R, i, so, sr, si, expr in STRIDED_SCAN_VIEWS:
        log("report: strided cumsum %s" % name)
        out = torch.empty(o * R * i, dtype=torch.float32, device=dev)

        def call():
            rd.rd_cumsum_strided(x, o, R, i, so, sr, si, False, out=out)

        reps = args.reps or 30
        ms = _median_ms(call, reps)
        nbytes = 8 * o * R * i
        plan = rd.rd_plan_cumsum_strided(cu, o, R, i, so, sr, si).as_dict()
        line = {"op": "cumsum", "view": name, "torch": expr, "shape": [o, R, i],
                "strides": [so, sr, si], "view_bytes": nbytes, "ms_median": round(ms, 5),
                "GBps": round(nbytes / ms / 1e6, 1),
                "frac_of_peak": round(nbytes / ms / 1e6 / PEAK_GBS, 4), "plan": plan,
                "reps": reps}
        if not args.no_oracle:
            v = np.lib.stride_tricks.as_strided(host, shape=(o, R, i),
                                                strides=(4 * so, 4 * sr, 4 * si),
                                                writeable=False)
            S, A = oracle.cumsum_dim(np.ascontiguousarray(v), o, R, i, False, threads)
            got = out.cpu().numpy().reshape(-1)
            line["parity"] = {"ok": bool(oracle.within_tolerance(got, S.reshape(-1),
                                                                 A.reshape(-1)).all())}
            del S, A, got
        print(json.dumps(line), flush=True)
        del out
    return 0


def _median_ms(fn, reps):
    """Median of `reps` event-timed calls of fn (the GPU kept busy while the
    host enqueues each call)."""
    import torch

    fn()
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        torch.cuda._sleep(200_000)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        ms.append(a.elapsed_time(b))
    ms.sort()
    return ms[len(ms) // 2]


def report_scan(args, dev, cu):
    """One JSON line per cumulative sum (both directions): GPU time warm and
    cold, GB/s over the algorithmic bytes (every element read once and written
    once), the oracle's host time, parity on every output."""
    import numpy as np
    import torch

    import oracle
    import sum_reduction_amd as rd
    import workloads

    threads = oracle.default_threads()
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    todo = list(workloads.SCAN_WORKLOADS.values())
    for spec in args.scan_shape or []:
        o, r, i = (int(v) for v in spec.lower().split("x"))
        todo.append(workloads.Workload("scan_%dx%dx%d" % (o, r, i), (o, r, i), o, r, i,
                                       "uniform", seed=0))
    for w in todo:
        host = workloads.generate(w)
        x = torch.from_numpy(host).to(dev)
        out = torch.empty_like(x)
        nbytes = 8 * w.numel
        # context, same bytes: a plain device copy (the read + write stream's
        # practical ceiling) and, for the problem 91 rows, the pages' library
        # formulation, cumsum of the flipped rows flipped back
        ctx = {"copy_ms": round(_median_ms(lambda: out.copy_(x), 20), 5)}
        if w.name in workloads.SCAN_WORKLOADS:
            xv = x.view(w.outer, w.R)
            ctx["torch_flip_cumsum_flip_ms"] = round(
                _median_ms(lambda: torch.cumsum(xv.flip(1), 1).flip(1), 5), 5)
            ctx["torch_cumsum_ms"] = round(
                _median_ms(lambda: torch.cumsum(xv, 1, out=out.view(w.outer, w.R)), 5), 5)
        print(json.dumps({"workload": w.name, "op": "context", "algorithmic_bytes": nbytes,
                          **ctx}), flush=True)
        for rev in (True, False):
            log("report: cumsum %s reverse=%d" % (w.name, rev))

            def call():
                rd.rd_cumsum_dim(x, w.outer, w.R, w.inner, reverse=rev, out=out)

            for _ in range(3):
                call()
            torch.cuda.synchronize()
            reps = args.reps or (50 if nbytes >= (1 << 30) else 500)

            def timed(cold):
                ms = []
                for _ in range(reps):
                    if cold:
                        flush.fill_(1.0)
                    torch.cuda._sleep(200_000)
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record()
                    call()
                    b.record()
                    b.synchronize()
                    ms.append(a.elapsed_time(b))
                ms.sort()
                med = ms[len(ms) // 2]
                return {"ms_median": round(med, 5), "ms_min": round(ms[0], 5),
                        "GBps_median": round(nbytes / med / 1e6, 1),
                        "frac_of_peak": round(nbytes / med / 1e6 / PEAK_GBS, 4)}

            warm, cold = timed(False), timed(True)
            plan = rd.rd_plan_cumsum(cu, w.outer, w.R, w.inner).as_dict()
            line = {"workload": w.name, "op": "cumsum", "reverse": rev, "shape": list(w.shape),
                    "algorithmic_bytes": nbytes, "warm": warm, "cold": cold, "reps": reps,
                    "plan": plan}
            if args.no_oracle:
                print(json.dumps(line), flush=True)
                continue
            got = out.cpu().numpy().reshape(w.outer, w.R * w.inner)
            # the oracle in blocks of outer indices (its fp64 outputs of the
            # whole array would not fit comfortably in host memory)
            blk = max(1, (1 << 25) // max(1, w.R * w.inner))
            ok, worst, cpu_s = True, 0.0, 0.0
            for o0 in range(0, w.outer, blk):
                o1 = min(w.outer, o0 + blk)
                part = host[o0 * w.R * w.inner:o1 * w.R * w.inner]
                t0 = time.perf_counter()
                S, A = oracle.cumsum_dim(part, o1 - o0, w.R, w.inner, rev, threads)
                cpu_s += time.perf_counter() - t0
                g = got[o0:o1].reshape(-1)
                ok &= bool(oracle.within_tolerance(g, S.reshape(-1), A.reshape(-1)).all())
                with np.errstate(invalid="ignore"):
                    r = np.abs(g.astype(np.float64) - S.reshape(-1)) / oracle.tolerance(
                        A.reshape(-1))
                worst = max(worst, float(np.nanmax(r)))
            line.update({
                "cpu_oracle": {"s": round(cpu_s, 4), "GBps": round(nbytes / cpu_s / 1e9, 3),
                               "threads": threads},
                "gpu_over_cpu": round(cpu_s * 1e3 / warm["ms_median"], 1),
                "parity": {"ok": ok, "max_err_over_tol": round(worst, 5)},
            })
            print(json.dumps(line), flush=True)
        del x, out, host
        torch.cuda.empty_cache()
    return 0


def report_one(w, op, host, x, out, flush, threads, cu, args):
    """One report line: workload `w` reduced with `op`, GPU warm and cold,
    the oracle's host time, parity."""
    import numpy as np
    import torch

    import oracle
    import sum_reduction_amd as rd

    nout = w.out_numel
    pair = op == "softmax_denom"
    # the softmax denominator writes two outputs (max, sum) per reduced column
    nbytes = w.in_bytes + 4 * nout * (2 if pair else 1)

    def call():
        if pair:
            if w.full_reduce:
                rd.rd_softmax_denom_1d(x, out[:1], out[1:2])
            else:
                rd.rd_softmax_denom_dim(x, w.outer, w.R, w.inner, out[:nout], out[nout:])
        elif w.full_reduce:
            rd.rd_reduce_1d(x, op, out=out[:1])
        else:
            rd.rd_reduce_dim(x, w.outer, w.R, w.inner, op, out=out[:nout])

    small = w.in_bytes < (1 << 30)
    reps = args.reps or (500 if small else 50)
    for _ in range(3):
        call()
    torch.cuda.synchronize()

    def timed(cold: bool):
        ms = []
        for _ in range(reps):
            if cold:
                flush.fill_(1.0)
            # keep the GPU busy while the host enqueues the call, so the
            # events see GPU time and not Python's enqueue latency
            torch.cuda._sleep(200_000)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            b.synchronize()
            ms.append(a.elapsed_time(b))
        ms.sort()
        return {"ms_median": round(ms[len(ms) // 2], 5), "ms_min": round(ms[0], 5),
                "ms_p90": round(ms[int(0.9 * (len(ms) - 1))], 5),
                "GBps_median": round(nbytes / ms[len(ms) // 2] / 1e6, 1),
                "frac_of_peak": round(nbytes / ms[len(ms) // 2] / 1e6 / PEAK_GBS, 4)}

    warm = timed(False)
    cold = timed(True)
    plan = (rd.rd_plan_reduce(cu, 1, w.numel, 1, op) if w.full_reduce
            else rd.rd_plan_reduce(cu, w.outer, w.R, w.inner, op)).as_dict()
    if args.no_oracle:
        return {"workload": w.name, "op": op, "shape": list(w.shape),
                "algorithmic_bytes": nbytes, "warm": warm, "cold": cold,
                "reps": reps, "plan": plan}
    got = out[:nout].cpu().numpy().reshape(-1)
    t0 = time.perf_counter()
    if pair:
        if w.full_reduce:
            M, S = oracle.softmax_denom_dim(host, 1, w.numel, 1)
        else:
            M, S = oracle.softmax_denom_dim(host, w.outer, w.R, w.inner, threads)
        A = S   # every term exp(x - c) is non-negative
        got_m, got = got, out[nout:].cpu().numpy().reshape(-1)
    elif w.full_reduce:
        S, A = oracle.reduce_1d(host, op)
        S, A = np.array([S]), np.array([A])
    else:
        S, A = oracle.reduce_dim(host, w.outer, w.R, w.inner, op, threads)
    cpu_s = time.perf_counter() - t0
    with np.errstate(invalid="ignore"):
        err = np.abs(got.astype(np.float64) - S.reshape(-1))
    tol = oracle.tolerance(A.reshape(-1))
    line = {
        "workload": w.name, "op": op, "shape": list(w.shape),
        "algorithmic_bytes": nbytes,
        "warm": warm, "cold": cold, "reps": reps, "plan": plan,
        "cpu_oracle": {"s": round(cpu_s, 4), "GBps": round(nbytes / cpu_s / 1e9, 3),
                       "threads": 1 if w.full_reduce else threads},
        "gpu_over_cpu": round(cpu_s * 1e3 / warm["ms_median"], 1),
        "parity": {"ok": bool(oracle.within_tolerance(got, S.reshape(-1),
                                                      A.reshape(-1)).all()),
                   "max_err_over_tol": round(float(np.nanmax(err / tol))
                                             if np.isfinite(err).any() else 0.0, 5)},
        "pages": PAGES_T4.get(w.name) if op == "sum" else None,
    }
    if op in ("max", "min"):  # exact reductions: the bits must match
        line["parity"]["bit_exact"] = bool(np.array_equal(
            got.view(np.uint32), S.reshape(-1).astype(np.float32).view(np.uint32)))
    if pair:  # the maxima are exact
        line["parity"]["max_bit_exact"] = bool(np.array_equal(
            got_m.view(np.uint32), M.reshape(-1).astype(np.float32).view(np.uint32)))
        line["parity"]["ok"] = line["parity"]["ok"] and line["parity"]["max_bit_exact"]
    if w.name == "harmonic_1e6" and op == "sum":
        line["harmonic_closed_form"] = float(
            np.log(w.numel) + 0.5772156649015329 + 1 / (2 * w.numel)
            - 1 / (12 * w.numel ** 2))
        line["gpu_value"] = float(got[0])
    return line


if __name__ == "__main__":
    sys.exit(main())
