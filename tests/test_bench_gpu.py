"""bench.py's output contract on the GPU: a short run of the headline leg and the CPU baseline
prints one JSON line with every field the benchmark promises."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_contract():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("bench.py --legs fwd,cpu --steps 3 --warmup 1 --cpu-seconds 1", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--legs", "fwd,cpu", "--steps", "3",
                        "--warmup", "1", "--cpu-seconds", "1"], capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 3 and out["warmup"] == 1
    assert out["value"] > 0 and out["ms_per_step"] > 0 and out["higher_is_better"] is True
    assert "8192" in out["config"]["workload"]
    rf = out["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and 0 < rf["frac"] < 1
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # TFLOP/s = flops / time
    assert abs(out["value"] - rf["algorithmic_flops_per_launch"] / (out["ms_per_step"] * 1e-3) / 1e12) < 0.01 * out["value"]
    cb = out["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
