"""Host logic of bench.py: the HBM-traffic figures it reports come only from
counter runs of the same GEMM launch on the same kernel sources."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

PLAN = {"tile_cfg": 0, "split": 1, "chunks_per_window": 4, "ring": 0, "windows": 4}


def _write(tmp_path, monkeypatch, **over):
    d = {"kernel_source_sha": "abc", "workload": "w", "precision": "exact", "a_format": "e4m3",
         "b_format": "e4m3", "ring": "events", "plan": {"tile_cfg": 0, "split": 1, "chunks_per_window": 4},
         "hbm_bytes_per_launch": 123}
    d.update(over)
    os.makedirs(tmp_path / "profiles", exist_ok=True)
    with open(tmp_path / "profiles" / "mxgemm_traffic_w_exact.json", "w") as f:
        json.dump(d, f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))


def test_traffic_matches_only_the_same_launch(tmp_path, monkeypatch):
    _write(tmp_path, monkeypatch)
    assert bench.load_traffic("w", "exact", "e4m3", "e4m3", "events", PLAN, "abc") == 123
    assert bench.load_traffic("w", "exact", "e4m3", "e4m3", "events", PLAN, "other") is None
    assert bench.load_traffic("w", "native", "e4m3", "e4m3", "events", PLAN, "abc") is None
    assert bench.load_traffic("w", "exact", "e5m2", "e4m3", "events", PLAN, "abc") is None
    assert bench.load_traffic("w", "exact", "e4m3", "e4m3", "flags", PLAN, "abc") is None
    assert bench.load_traffic("w", "exact", "e4m3", "e4m3", "events", dict(PLAN, split=2), "abc") is None
    assert bench.load_traffic("x", "exact", "e4m3", "e4m3", "events", PLAN, "abc") is None


def test_traffic_files_in_tree_name_their_launch():
    """Every committed traffic file records the kernel sources, mode,
    formats, ring and plan it was counted on, and the summary it came from."""
    prof = os.path.join(ROOT, "profiles")
    files = [f for f in os.listdir(prof) if f.startswith("mxgemm_traffic_")]
    assert files
    for name in files:
        with open(os.path.join(prof, name)) as f:
            d = json.load(f)
        for key in ("kernel_source_sha", "precision", "a_format", "b_format", "ring", "plan",
                    "hbm_bytes_per_launch", "source"):
            assert key in d, (name, key)
        assert name == f"mxgemm_traffic_{d['workload']}_{d['precision']}.json"
        assert os.path.exists(os.path.join(ROOT, d["source"]))


def test_more_than_one_gpu_is_refused():
    """bench.py runs on one GPU: --gpus N > 1 exits with a message before
    touching a device."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_roofline_against_the_metric_peak():
    """The GEMM roofline of an MFMA-bound workload is priced against the
    MX-FP8 peak the metric names, with the contraction's own MFMA peak
    beside it; a skinny launch below the ridge point is priced against HBM."""
    from mxfp8_block_scaled_mxgemm_amd import inputs
    w = inputs.WORKLOADS["outlier_m8192_n8192_k8192"]
    r = bench.gemm_roofline(w, {"windows": 4}, 0.2, "exact", False)
    assert r["bound"] == "mfma" and r["peak"] == 5000.0 and r["unit"] == "TFLOP/s"
    flops = 2 * 2048 * 8192 * 8192
    assert abs(r["achieved"] - flops / 2e-4 / 1e12) < 1e-2
    assert abs(r["frac"] - flops / 2e-4 / 1e12 / 5000.0) < 1e-4
    assert r["kernel_mfma_peak"] == 2500.0
    assert abs(r["frac_of_kernel_mfma_peak"] - 2 * r["frac"]) < 1e-3
    s = inputs.WORKLOADS["skinny_m64_n2048_k7168"]
    r = bench.gemm_roofline(s, {"windows": 2}, 0.01, "exact", False)
    assert r["bound"] == "hbm" and r["peak"] == 8000.0
    nbytes = (32 * 7168 + 2048 * 7168) * 33 / 32 + 32 * 2048 * 2
    assert abs(r["achieved"] - nbytes / 1e-5 / 1e9) < 1e-2
