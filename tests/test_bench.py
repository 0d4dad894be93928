"""The bench.py contract: one JSON line with the metric, the value, the
roofline block and the CPU baseline (on a GPU), and a clear refusal of more
than one GPU or of a host without one (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(args, env=None, timeout=600):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          env=e, timeout=timeout, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    for args, env in ((["--gpus", "2"], None), (["--gpus", "8"], None), ([], {"WORLD_SIZE": "2"})):
        r = _run(args, env)
        assert r.returncode == 2, (args, r.stdout, r.stderr)
        assert "one GPU" in r.stderr and r.stdout == ""


def _has_gpu():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="a GPU is visible")
def test_no_gpu_is_refused():
    r = _run(["--steps", "1", "--warmup", "0"])
    assert r.returncode == 2 and "needs a GPU" in r.stderr and r.stdout == ""


@pytest.mark.gpu
def test_json_line():
    r = _run(["--steps", "3", "--warmup", "1", "--no-ceiling", "--workload", "harmonic_1e6",
              "--workload", "uniform_1e8"])
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key, kind in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                      ("steps", int), ("warmup", int), ("ms_per_step", float),
                      ("higher_is_better", bool), ("scaling", str), ("dtype", str),
                      ("data", str), ("config", dict), ("roofline", dict),
                      ("cpu_baseline", dict)):
        assert isinstance(d[key], kind), key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "GB/s" and d["value"] > 0 and d["vs_baseline"] is None
    assert d["config"]["workload"] == "harmonic_1e6 + uniform_1e8"
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert "traffic" in rf and rf["workload"] == "uniform_1e8"
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    # each leg reported with the threads it ran on: both are full reduces,
    # the oracle's sequential loop
    assert set(cb["legs"]) == {"harmonic_1e6", "uniform_1e8"}
    assert all(leg["threads"] == 1 and leg["GBps"] > 0 for leg in cb["legs"].values())
    assert d["parity"]["ok"] is True
