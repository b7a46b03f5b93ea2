"""Build-time properties of the gfx950 kernels (cross-compiled here, no GPU):
no GEMM or staging kernel spills registers to scratch, and the large exact
kernel fits one work-group per CU with two LDS stages."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp8_block_scaled_mxgemm_amd", "csrc")


def _resource_usage(src):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    from mxfp8_block_scaled_mxgemm_amd import build
    cmd = [hipcc, "-x", "hip", *build.HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-c", os.path.join(CSRC, src), "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels = {}
    name = None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?:\s*\[[^\]]*\])?: (\d+)", line)
        if m and name:
            kernels[name][m.group(1).strip()] = int(m.group(2))
    return kernels


def test_gemm_kernels_do_not_spill():
    kernels = _resource_usage("gemm_e4m3_e4m3.hip")
    gemm = {k: v for k, v in kernels.items() if "mxgemm" in k}
    assert len(gemm) >= 10, sorted(kernels)
    for k, v in gemm.items():
        assert v.get("VGPRs Spill", 0) == 0 and v.get("SGPRs Spill", 0) == 0, (k, v)
        assert v.get("ScratchSize", 0) == 0, (k, v)
    exact = [v for k, v in gemm.items() if "mxgemm_exact_kernelILi256ELi256E" in k]
    assert len(exact) == 1
    assert exact[0]["LDS Size"] <= 160 * 1024 and exact[0]["Occupancy"] == 1


def test_staging_and_ring_kernels_do_not_spill():
    for src in ("kernels.hip", "ring.hip"):
        for k, v in _resource_usage(src).items():
            assert v.get("VGPRs Spill", 0) == 0 and v.get("ScratchSize", 0) == 0, (src, k, v)
