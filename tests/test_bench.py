"""bench.py's contract: one JSON line with the metric, the step timing, the
roofline of the fused kernel and the CPU oracle baseline; N above 1 refused.

The GPU test runs the benchmark in a child process on a short workload (the
cross-attention shape, a few steps) exactly as the driver runs it."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, BENCH, "--gpus", "2"], stdout=subprocess.PIPE,
                         stderr=subprocess.PIPE, text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_prints_one_json_line():
    print("  launch bench.py --workload text_cross --steps 3 --warmup 1", flush=True)
    res = subprocess.run([sys.executable, BENCH, "--workload", "text_cross", "--steps", "3",
                          "--warmup", "1", "--cpu-seconds", "3"], stdout=subprocess.PIPE,
                         stderr=subprocess.PIPE, text=True, timeout=600, cwd=ROOT)
    print(res.stderr[-2000:], flush=True)
    assert res.returncode == 0
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "TFLOP/s" and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["higher_is_better"] is True and d["dtype"] == "bf16"
    assert isinstance(d["config"]["workload"], str) and d["config"]["Nk"] == 512
    r = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in r, key
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2516.6
    assert abs(r["frac"] - r["achieved"] / r["peak"]) <= 1e-4
    # the fused kernel alone is faster than the whole step (pack included)
    assert r["achieved"] >= d["value"] * 0.999
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "TFLOP/s" and c["value"] > 0
    assert c["cores"] == len(os.sched_getaffinity(0)) and c["sample"]
