"""bench.py end to end on the GPU: one JSON line with the fields the report
is read from, on a small workload (run as a child process)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_json_line_small_workload():
    print("[bench] tiny_m128_n256_k512, 3 steps", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "tiny_m128_n256_k512",
                        "--steps", "3", "--warmup", "1", "--warmup-ms", "2", "--no-cpu-baseline",
                        "--telemetry-seconds", "0"],
                       capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["unit"] == "TFLOP/s"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    ro = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in ro, key
    assert ro["bound"] in ("hbm", "mfma") and 0 < ro["frac"] <= 1
    assert d["config"]["workload"].startswith("tiny_m128_n256_k512")
    # value is the whole step: 2 M N K over the mean step time
    assert abs(d["value"] - d["config"]["flop_per_step"] / (d["ms_per_step"] * 1e-3) / 1e12) < 1e-2 * d["value"]
