"""bench.py: refuses more than one GPU (this library has no multi-GPU path),
and prints one JSON line of the documented shape."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


@pytest.mark.gpu
def test_bench_json_line():
    """A short bench run prints one JSON line with the contract's fields, a
    positive step rate, and a roofline whose fraction is achieved / peak."""
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "3",
                        "--no-cpu-baseline", "--no-supplementary"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [ln for ln in p.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 3 and out["warmup"] == 3
    assert out["value"] > 0 and out["ms_per_step"] > 0
    assert "workload" in out["config"]
    r = out["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert 0 < r["frac"] < 1 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    # value is the step's flops over the step's wall time
    assert abs(out["value"] - out["config"]["attn_flops_per_step"] / (out["ms_per_step"] * 1e-3) / 1e12) \
        < 1e-6 * out["value"]
