"""Build-time properties of the gfx950 device code (cross-compiled here, no
GPU), from one parallel compile of every source to assembly:
- memory is written only through vector instructions: no scalar-cache
  store, atomic, write-back or discard appears anywhere;
- no kernel spills registers to scratch (and the GEMM kernels spill none
  at all), and the exact GEMM kernels (256 x 128 on eight waves, 128 x 128
  on four and 64 x 64 in four K groups, with fresh and running FP32
  accumulators) fit a CU at one work-group; no 256 x 256 exact kernel is
  built.
This file is CPU-only and is not sent to GPU runs."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp8_block_scaled_mxgemm_amd", "csrc")
SOURCES = ["kernels.hip", "ring.hip", "gemm_e4m3_e4m3.hip", "gemm_e5m2_e5m2.hip",
           "gemm_e4m3_e5m2.hip", "gemm_e5m2_e4m3.hip"]
SCALAR_WRITES = re.compile(r"^\s+s_(store|atomic|dcache_wb|dcache_discard|buffer_store|scratch_store)",
                           re.MULTILINE)


@pytest.fixture(scope="module")
def compiled(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    from mxfp8_block_scaled_mxgemm_amd import build
    d = tmp_path_factory.mktemp("isa")
    procs = {}
    for src in SOURCES:
        cmd = [hipcc, "-x", "hip", *build.HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(d / (src + ".s")),
               "-Rpass-analysis=kernel-resource-usage"]
        procs[src] = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    out = {}
    for src, p in procs.items():
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, err[-2000:]
        out[src] = ((d / (src + ".s")).read_text(), _resource_usage(err))
    return out


def _resource_usage(remarks):
    kernels, name = {}, None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?:\s*\[[^\]]*\])?: (\d+)", line)
        if m and name:
            kernels[name][m.group(1).strip()] = int(m.group(2))
    return kernels


@pytest.mark.parametrize("src", SOURCES)
def test_no_scalar_cache_writes(compiled, src):
    asm, _ = compiled[src]
    assert "global_" in asm
    hits = SCALAR_WRITES.findall(asm)
    assert not hits, f"{src}: scalar-cache writes {sorted(set(hits))}"


@pytest.mark.parametrize("src", SOURCES)
def test_no_register_spills(compiled, src):
    _, kernels = compiled[src]
    assert kernels
    for k, v in kernels.items():
        # SGPR spills go to VGPR lanes (the persistent ring kernel has some);
        # nothing may go to scratch memory
        assert v.get("VGPRs Spill", 0) == 0 and v.get("ScratchSize", 0) == 0, (k, v)
        if "mxgemm" in k:
            assert v.get("SGPRs Spill", 0) == 0, (k, v)


def test_exact_kernels_fit_one_work_group_per_cu(compiled):
    """256 x 128 runs eight waves (two per SIMD), 128 x 128 four (one per
    SIMD), 64 x 64 four K groups of one wave (one per SIMD); either way one
    work-group fills a CU's LDS share and SIMDs."""
    _, kernels = compiled["gemm_e4m3_e4m3.hip"]
    assert not [k for k in kernels if "mxgemm_exact_kernelILi256ELi256E" in k]
    for tile, waves_per_simd in (("ILi256ELi128ELi4ELi2ELi1E", 2), ("ILi128ELi128ELi2ELi2ELi1E", 1),
                                 ("ILi64ELi64ELi1ELi1ELi4E", 1)):
        exact = [v for k, v in kernels.items() if "mxgemm_exact_kernel" + tile in k]
        assert len(exact) == 1, tile
        assert exact[0]["LDS Size"] <= 160 * 1024 and exact[0]["Occupancy"] == waves_per_simd, exact[0]
