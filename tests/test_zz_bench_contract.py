"""bench.py's command-line contract: one JSON line with the fields the harness reads.

The CPU test checks that more than one GPU is refused before anything touches a device.  The
GPU test runs a short bench on the tiny fp32 layer (c1) and checks the line's fields, their
types and the roofline and CPU-baseline objects.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)
    assert res.stdout.strip() == "" or not res.stdout.strip().startswith("{")


@pytest.mark.gpu
def test_bench_json_line():
    res = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--config", "c1", "--steps", "3",
                          "--warmup", "1", "--no-pair", "--cpu-seconds", "1"],
                         capture_output=True, text=True, timeout=240)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout[-2000:]
    out = json.loads(lines[0])
    for k, t in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                 ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                 ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(out[k], t), (k, out.get(k))
    assert out["n_gpus"] == 1 and out["steps"] == 3 and out["warmup"] == 1
    assert out["value"] > 0 and out["ms_per_step"] > 0 and out["vs_baseline"] is None
    assert out["config"]["workload"].startswith("c1")
    roof = out["roofline"]
    assert roof["bound"] in ("hbm", "mfma", "alu") and roof["unit"] in ("GB/s", "TFLOP/s")
    assert roof["peak"] > 0 and 0 < roof["achieved"] and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert "traffic" in roof
    assert roof["kernel"].startswith("grouped_ffn_kernel<float")
    st = out["step_ms"]
    assert st["reps"] >= 50 and 0 < st["min_ms"] <= st["median_ms"] <= st["max_ms"]
    cpu = out["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert cpu["usable_cpus"] >= 1 and "cpu_model" in cpu
    assert cpu["c1_one_thread"]["threads"] == 1 and cpu["c1_one_thread"]["tokens_per_s"] > 0
