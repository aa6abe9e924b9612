"""The benchmark's output contract: `bench.py` (short settings) prints one
JSON line with the metric, the whole-job value, the step time, the roofline
object of the dominant kernel and the CPU-baseline field, and refuses more
than one GPU."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_its_fields():
    p = subprocess.run([sys.executable, BENCH, "--steps", "3", "--warmup", "1", "--step-only", "--no-configs",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [ln for ln in p.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for key, kind in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                      ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                      ("dtype", str), ("data", str), ("config", dict), ("roofline", dict)):
        assert isinstance(d[key], kind), (key, d.get(key))
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert abs(d["value"] - d["config"]["tokens"] / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]
    assert d["config"]["workload"] == "llama8b_128k" and "model" not in d["config"]
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma", "alu") and r["unit"] in ("GB/s", "TFLOP/s")
    assert r["achieved"] > 0 and r["peak"] > 0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    assert "cpu_baseline" in d and d["cpu_baseline"] is None   # skipped by --no-cpu-baseline


def test_bench_refuses_more_than_one_gpu():
    """Checked before anything touches a GPU, so it runs on the CPU too."""
    p = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert p.returncode != 0 and "single-GPU" in p.stderr
