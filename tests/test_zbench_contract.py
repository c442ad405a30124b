"""The benchmark's one-line JSON contract, on the launch-bound tiny workload (a few steps)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    print("[case] bench tiny_gpt_mlp", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny_gpt_mlp", "--steps", "3",
                        "--warmup", "2", "--rounds", "2", "--cpu-seconds", "0.5"], capture_output=True, text=True, timeout=300,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2 and d["value"] > 0
    assert d["config"]["workload"] == "tiny_gpt_mlp"
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["peak"] == 2500.0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    for k in ("hidden_copy_pct", "hidden_copy_pct_single_call", "hidden_copy_wall_pct"):
        assert d[k] is None or 0.0 <= d[k] <= 100.0, k
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0

