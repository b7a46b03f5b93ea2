"""Build the HIP library ``libmxgemm_seg.so`` for gfx950, in-tree.

    python -m mxfp8_block_scaled_mxgemm_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmxgemm_seg.so")

# One GEMM translation unit per (A, B) FP8 format pair, compiled in parallel.
SOURCES = ["kernels.hip", "gemm_e4m3_e4m3.hip", "gemm_e5m2_e5m2.hip", "gemm_e4m3_e5m2.hip",
           "gemm_e5m2_e4m3.hip", "ring.hip", "mxgemm_seg.cpp"]
ARCH = "gfx950"

# Packed-FP32 ALU forms are switched off for every kernel (the compiler would
# otherwise form them from ordinary float code).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# The benchmark's MFMA-rate probe, a library of its own (not the product).
PROBE_SOURCE = "mfma_rate.hip"
PROBE_LIB = os.path.join(PKG, "libmxgemm_rate.so")


def build_probe(verbose: bool = False) -> str:
    cmd = [hipcc(), "-x", "hip", *HIP_FLAGS, "-shared", "-o", PROBE_LIB + ".tmp",
           os.path.join(CSRC, PROBE_SOURCE)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on " + PROBE_SOURCE)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library (and the benchmark's
    MFMA-rate probe); always rebuilds."""
    objs = []
    tmpdir = os.path.join(PKG, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    procs = []
    for src in SOURCES:
        obj = os.path.join(tmpdir, src + ".o")
        cmd = [hipcc(), "-x", "hip", *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        while sum(p.poll() is None for _, p in procs) >= jobs:
            procs[[p.poll() is None for _, p in procs].index(True)][1].wait()
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out)
            failed.append(src)
        elif verbose and out:
            sys.stderr.write(out)
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    build_probe(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
