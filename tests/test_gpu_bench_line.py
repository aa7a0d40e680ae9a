"""The benchmark's output contract on a GPU: one run of bench.py on the small
fp32 workload (as a child process, the way the benchmark is started) prints one
JSON line carrying every field the line promises, with consistent values."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(300)
def test_bench_prints_one_complete_json_line():
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "tiny_fp32",
           "--steps", "3", "--warmup", "1", "--no-cpu-baseline"]
    print("[bench line] " + " ".join(cmd[2:]), file=sys.stderr, flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "plan_gather_combine", "stages_us"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["config"]["workload"] == "tiny_fp32" and d["dtype"] == "f32"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # value is routed rows per second of the timed steps
    rows = d["config"]["T"] * d["config"]["top_k"]
    assert abs(d["value"] * d["ms_per_step"] * 1e-3 / rows - 1) < 1e-6
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] in ("hbm", "mfma") and roof["achieved"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    same = roof["read_probe_same_bytes"]
    assert same["bytes"] >= roof["algorithmic_bytes_per_launch"] and same["gbs"] > 0
    assert "cpu_baseline" not in d
