"""The benchmark's output contract: one JSON line with the fields a driver
reads (metric, value, unit, n_gpus, steps, warmup, ms_per_step, ...), the
roofline object of the dominant kernel and the workload description, and a
refusal of more than one GPU.  The GPU case runs the tiny workload (1 head,
64 + 1,024 + 64 tokens) for a few steps in a child process."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    text = r.stdout + r.stderr
    assert "one GPU" in text, text
    assert not any(l.startswith("{") for l in r.stdout.splitlines()), r.stdout


@pytest.mark.gpu
def test_tiny_workload_json_line():
    print("[bench contract] tiny workload, 3 steps", flush=True)
    r = subprocess.run([sys.executable, BENCH, "--workload", "tiny", "--steps", "3", "--warmup", "1",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key, kind in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                      ("steps", int), ("warmup", int), ("ms_per_step", float),
                      ("higher_is_better", bool), ("scaling", str), ("dtype", str), ("data", str),
                      ("config", dict), ("roofline", dict)]:
        assert isinstance(d[key], kind), (key, d.get(key))
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["unit"] == "TFLOP/s" and d["dtype"] == "bf16"
    assert d["config"]["workload"].startswith("tiny")
    assert d["config"]["k"] == 3
    roof = d["roofline"]
    assert roof["bound"] in ("hbm", "mfma", "alu") and roof["unit"] in ("GB/s", "TFLOP/s")
    assert 0 < roof["frac"] < 1 and roof["achieved"] > 0 and roof["peak"] == 2500.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    assert "vs_baseline" in d and "traffic" in roof
