#!/usr/bin/env python3
"""Benchmark of the segmented MXFP8 GEMM on one MI355X.

One step = one whole pass of the hot path over one batch of synthetic input:
staging of every chunk of every rank segment through the ring, the
block-scaled GEMM over all windows (with split-K fix-up where planned) and
the bfloat16 epilogue -- one ``mxgemm_seg_run`` call.  Inputs are quantised
on the GPU before timing and are resident in HBM.  Before every timed step a
512 MiB buffer is written to push A, B and C out of L2 and the MALL.  Each
timed loop is preceded by untimed steps of the same kind: at least --warmup
steps and --warmup-ms of GPU time.

Prints ONE JSON line (rank 0 / the only rank):
  value      = 2*M*N*K / mean step time (steps issued on the stream), in
               TFLOP/s, for the headline workload (--config, default the
               8192-cube outlier workload); the mean over replays of a HIP
               graph of the step is reported beside it
  roofline   = the GEMM kernel's algorithmic FLOP (or bytes, below the ridge
               point) per launch / its mean launch duration (HIP events
               around each launch, on its stream), against the MI355X dense
               MX-FP8 MFMA peak (the metric's peak; the bf16 MFMA peak of the
               exact mode's contraction beside it) or HBM
  configs    = the same figures for the other workloads (stream timer, and
               the mean over replays of a HIP graph of the step beside it)
  measured_peaks = an MFMA-rate probe (scaled FP8 and bf16) and a device copy
               of 1 GiB, the measured denominators beside the published ones
  cpu_baseline = the CPU oracle on a bounded row sample of the headline
               workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MXFP8 segmented GEMM TFLOP/s and % of MI355X MX-FP8 MFMA peak"
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 / MXFP8 MFMA
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense BF16 MFMA (the exact mode's contraction)
PEAK_HBM_GBS = 8000.0
FLUSH_BYTES = 512 << 20


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# Sources the GEMM kernels are built from (the host library and the other
# kernels are not part of it): a counter summary stays valid while these
# are unchanged.
GEMM_SOURCES = ("device_util.h", "gemm_impl.h", "kernels.h", "schedule.h", "gemm_e4m3_e4m3.hip",
                "gemm_e5m2_e5m2.hip", "gemm_e4m3_e5m2.hip", "gemm_e5m2_e4m3.hip")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mxfp8_block_scaled_mxgemm_amd", "csrc")
    for name in GEMM_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, precision: str, a_format: str, b_format: str, ring: str, plan: dict,
                 sha: str):
    """HBM bytes per GEMM launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel sources for the same GEMM launch
    (precision mode, operand formats, ring protocol, tile configuration,
    split and window)."""
    path = os.path.join(ROOT, "profiles", f"mxgemm_traffic_{workload}_{precision}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != sha:
        return None
    if (d.get("precision"), d.get("a_format"), d.get("b_format"), d.get("ring")) != (
            precision, a_format, b_format, ring):
        return None
    if d.get("plan") != {k: plan[k] for k in ("tile_cfg", "split", "chunks_per_window")}:
        return None
    return d.get("hbm_bytes_per_launch")


# Telemetry: a child process (started before this process touches the GPU)
# polls amd-smi for the shader clocks of the XCDs and the socket power and
# appends one JSON line per sample to a file.
SAMPLER = r"""
import json, os, subprocess, sys, time
out, parent = sys.argv[1], int(sys.argv[2])
use_temp = True
while True:
    try:
        os.kill(parent, 0)
    except OSError:
        break
    if os.path.exists(out + ".stop"):
        break
    try:
        cmd = ["amd-smi", "metric", "-g", "0", "--clock", "--power", "--json"]
        if use_temp:
            cmd.insert(-1, "--temperature")
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=10)
        if r.returncode != 0 and use_temp:
            use_temp = False
            continue
        g = json.loads(r.stdout)["gpu_data"][0]
        num = lambda v: v if isinstance(v, (int, float)) else None
        clk = [v["clk"]["value"] for k, v in g["clock"].items()
               if k.startswith("gfx_") and isinstance(v.get("clk", {}).get("value"), (int, float))]
        mem = num(((g["clock"].get("mem_0") or {}).get("clk") or {}).get("value"))
        pw = g["power"]["socket_power"]["value"]
        temp = None
        for key in ("hotspot", "edge"):
            t = (g.get("temperature") or {}).get(key)
            t = t.get("value") if isinstance(t, dict) else t
            if num(t) is not None:
                temp = t
                break
        with open(out, "a") as f:
            f.write(json.dumps({"t": time.time(), "gfx_mhz": clk, "power_w": pw, "mem_mhz": mem,
                                "temp_c": temp}) + "\n")
    except Exception:
        time.sleep(0.5)
    time.sleep(0.1)
"""


def start_sampler(path: str):
    import shutil
    import subprocess
    if shutil.which("amd-smi") is None:
        return None
    for f in (path, path + ".stop"):
        if os.path.exists(f):
            os.remove(f)
    return subprocess.Popen([sys.executable, "-c", SAMPLER, path, str(os.getpid())],
                            stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)


def read_samples(path: str, t0: float, t1: float):
    if not os.path.exists(path):
        return []
    rows = []
    with open(path) as f:
        for line in f:
            try:
                d = json.loads(line)
            except ValueError:
                continue
            if t0 <= d["t"] <= t1 and d["gfx_mhz"]:
                rows.append(d)
    return rows


def cpu_baseline(w, target_s: float):
    """Time the CPU oracle (as it stands) on the first rows of C."""
    import numpy as np
    import oracle
    from mxfp8_block_scaled_mxgemm_amd import inputs
    a32, b32 = inputs.fp32_operands(w)
    qa, sa = oracle.quantize_mxfp8(a32)
    qb, sb = oracle.quantize_mxfp8(b32)
    a_seg, s_seg = inputs.split_segments(qa, w.R), inputs.split_segments(sa, w.R)
    del a32, b32, qa, sa
    threads = oracle.num_threads()
    rows = max(1, threads // 2)
    t0 = time.perf_counter()
    oracle.mxgemm_seg_rows(a_seg, s_seg, qb, sb, 0, rows)
    dt = time.perf_counter() - t0
    rows = int(min(w.M, max(rows, rows * target_s / max(dt, 1e-3))))
    rows = max(threads, (rows // threads) * threads) if rows >= threads else rows
    t0 = time.perf_counter()
    oracle.mxgemm_seg_rows(a_seg, s_seg, qb, sb, 0, rows)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"rows [0, {rows}) of C = {rows}x{w.N} outputs at K={w.K} "
                      f"(dequantise + double-precision dot + bfloat16 rounding), {dt:.1f} s "
                      f"on {threads} threads of {cpu}"}


def gemm_roofline(w, plan, gemm_ms_per_launch, precision, ring_flags):
    """Roofline of the GEMM kernel for one workload: achieved FLOP/s (or
    bytes/s below the ridge point) per launch against the MX-FP8 peak (the
    metric's; the contraction's own MFMA peak beside it) or HBM."""
    launches = 1 if ring_flags else plan["windows"]
    flops_per_launch = float(w.flops) / launches
    rows_w = w.M / launches
    # algorithmic bytes of one GEMM launch: A rows and B with their E8M0
    # scales, C in bfloat16
    bytes_per_launch = (rows_w * w.K + w.N * w.K) * 33 / 32 + rows_w * w.N * 2
    kernel_peak = PEAK_BF16_TFLOPS if precision == "exact" else PEAK_FP8_TFLOPS
    hbm_bound = flops_per_launch / bytes_per_launch < PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    tflops = flops_per_launch / (gemm_ms_per_launch * 1e-3) / 1e12
    gbs = bytes_per_launch / (gemm_ms_per_launch * 1e-3) / 1e9
    r = {"bound": "hbm" if hbm_bound else "mfma"}
    if hbm_bound:
        r.update(achieved=round(gbs, 3), peak=PEAK_HBM_GBS, unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4))
    else:
        r.update(achieved=round(tflops, 3), peak=PEAK_FP8_TFLOPS, unit="TFLOP/s",
                 frac=round(tflops / PEAK_FP8_TFLOPS, 4))
    r.update(gemm_tflops=round(tflops, 3), gemm_gbs=round(gbs, 2),
             frac_of_mxfp8_peak=round(tflops / PEAK_FP8_TFLOPS, 4),
             kernel_mfma=("bf16 (exact products, v_mfma_f32_*_bf16)" if precision == "exact"
                          else "scaled FP8 (v_mfma_scale_f32_*_f8f6f4)"),
             kernel_mfma_peak=kernel_peak,
             frac_of_kernel_mfma_peak=round(tflops / kernel_peak, 4),
             frac_of_hbm=round(gbs / PEAK_HBM_GBS, 4),
             bytes_per_launch=int(bytes_per_launch), flops_per_launch=int(flops_per_launch),
             gemm_us_per_launch=round(gemm_ms_per_launch * 1e3, 3), launches_per_step=launches)
    return r


def measured_peaks(torch, dev, stream):
    """Measured denominators: the MFMA-rate probe (scaled FP8 and bf16, no
    memory traffic) and a 1 GiB device-to-device copy."""
    import ctypes
    out = {}
    lib_path = os.path.join(ROOT, "mxfp8_block_scaled_mxgemm_amd", "libmxgemm_rate.so")
    if os.path.exists(lib_path):
        lib = ctypes.CDLL(lib_path)
        lib.mxgemm_probe_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_void_p, ctypes.c_void_p]
        lib.mxgemm_probe_mfma_rate.restype = ctypes.c_int
        grid, iters = 2048, 512
        buf = torch.empty(grid * 256, dtype=torch.float32, device=dev)
        for kind, name, flop in ((0, "scaled_fp8_mfma_tflops", 131072), (1, "bf16_mfma_tflops", 32768)):
            def launch():
                rc = lib.mxgemm_probe_mfma_rate(kind, grid, iters, ctypes.c_void_p(buf.data_ptr()),
                                                ctypes.c_void_p(stream.cuda_stream))
                if rc != 0:
                    raise RuntimeError(f"MFMA probe launch failed ({rc})")
            for _ in range(3):
                launch()
            times = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                launch()
                e1.record(stream)
                e1.synchronize()
                times.append(e0.elapsed_time(e1))
            total = grid * 4 * iters * 16 * flop          # waves x MFMAs x FLOP
            out[name] = round(total / (statistics.median(times) * 1e-3) / 1e12, 1)
        out["mfma_probe"] = (f"{grid} work-groups x 4 waves, each {iters * 16} back-to-back MFMAs on "
                             "4 independent accumulators, no memory traffic; median of 5 launches")
        del buf
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1.0)
    for _ in range(2):
        dst.copy_(src)
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    nbytes = 2 * src.numel() * 4
    out["copy_gbs"] = round(nbytes / (statistics.median(times) * 1e-3) / 1e9, 1)
    out["copy"] = "1 GiB device-to-device copy (read + write bytes / time), median of 5"
    del src, dst

    # floors for short steps: the event-to-event time of a one-element fill
    # (a launch that does nothing else), and of a copy moving the skinny
    # workload's algorithmic bytes (read + write), caches flushed first
    def floor_us(fn, reps=20):
        flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        ts = []
        for _ in range(reps):
            flush.fill_(0.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        del flush
        return round(statistics.median(ts), 2)

    one = torch.empty(1, dtype=torch.float32, device=dev)
    out["empty_launch_us"] = floor_us(lambda: one.fill_(0.0))
    from mxfp8_block_scaled_mxgemm_amd import inputs
    skinny = inputs.WORKLOADS["skinny_m64_n2048_k7168"]
    half = skinny.algorithmic_bytes // 2 // 4
    a, b = torch.empty(half, dtype=torch.float32, device=dev), torch.empty(half, dtype=torch.float32, device=dev)
    a.fill_(1.0)
    out["skinny_bytes_copy_us"] = floor_us(lambda: b.copy_(a))
    out["floors"] = (f"event-to-event medians of 20 after a 512 MiB flush: a one-element fill, and a "
                     f"copy of {2 * half * 4} bytes read + written (the skinny workload's "
                     f"{skinny.algorithmic_bytes} algorithmic bytes)")
    del a, b, one
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5,
                    help="untimed steps before each timed loop (at least; see --warmup-ms)")
    ap.add_argument("--warmup-ms", type=float, default=25.0,
                    help="untimed GPU time before each timed loop, in steps of the same kind "
                         "(at most 200 steps)")
    ap.add_argument("--config", default="outlier_m8192_n8192_k8192", help="headline workload (default outlier_m8192_n8192_k8192)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload block for the other workloads")
    ap.add_argument("--config-steps", type=int, default=20,
                    help="timed steps per workload in the per-workload block")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=25.0)
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--telemetry-seconds", type=float, default=2.0,
                    help="sustained replays while amd-smi samples the shader clock (0: off)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the second timer (replays of one HIP-graph-captured step)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured denominators")
    ap.add_argument("--tile-cfg", type=int, default=-1)
    ap.add_argument("--split", type=int, default=-1)
    ap.add_argument("--window", type=int, default=-1)
    ap.add_argument("--ring", choices=["auto", "events", "flags"], default="auto",
                    help="ring protocol (default: the planner's choice)")
    ap.add_argument("--precision", choices=["exact", "native"], default="exact",
                    help="GEMM arithmetic (default exact: parity-green on every workload)")
    ap.add_argument("--a-format", choices=["e4m3", "e5m2"], default="e4m3",
                    help="FP8 format of the A codes")
    ap.add_argument("--b-format", choices=["e4m3", "e5m2"], default="e4m3",
                    help="FP8 format of the B codes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 256 MiB device-to-device three times (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "copies": 3}))
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the ranks of this "
              "method are simulated as segments in one GPU's memory, and no multi-GPU path is "
              "built.", file=sys.stderr)
        sys.exit(2)

    tele_path = os.path.join("/tmp", f"mxgemm_bench_telemetry_{os.getpid()}.jsonl")
    sampler = start_sampler(tele_path) if args.telemetry_seconds > 0 else None

    import torch
    import mxfp8_block_scaled_mxgemm_amd as pkg
    from mxfp8_block_scaled_mxgemm_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pkg.load()                       # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    prec = pkg.PRECISION_EXACT if args.precision == "exact" else pkg.PRECISION_NATIVE
    fmts = (args.a_format, args.b_format)

    def make_inputs(w):
        a32, b32 = inputs.fp32_operands(w)
        a_d = torch.from_numpy(a32).to(dev)
        b_d = torch.from_numpy(b32).to(dev)
        del a32, b32
        a_q, a_s = pkg.quantize_segments(a_d, w.R, fmt=args.a_format)
        b_q, b_s = pkg.quantize_mxfp8(b_d, fmt=args.b_format)
        del a_d, b_d
        c = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        return a_q, a_s, b_q, b_s, c

    def flush_caches():
        if not args.no_flush:
            flush.fill_(1.0)

    warm_log = {}

    def warm_up(run_one, label):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n, spent = 0, 0.0
        while n < 200 and (n < max(1, args.warmup) or spent < args.warmup_ms):
            batch = max(1, min(8, 200 - n))
            ev0.record(stream)
            for _ in range(batch):
                flush_caches()
                run_one()
            ev1.record(stream)
            ev1.synchronize()
            spent += ev0.elapsed_time(ev1)
            n += batch
        warm_log[label] = {"steps": n, "ms": round(spent, 2)}

    # ---- timed steps ------------------------------------------------------
    # Each step is one run() of the whole path, issued on the stream the way
    # a caller of mxgemm_seg_run issues it; these K steps give `value`.  A
    # 512 MiB fill precedes every step (outside its events) so no step starts
    # with warm caches; the fill also keeps the host ahead of the GPU, so the
    # steps carry no host-enqueue gaps.  The same step captured once into a
    # HIP graph and replayed K times is timed too and reported beside it
    # (graph_ms_per_step; --no-graph skips it).
    def timed(run_one, steps):
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            flush_caches()
            starts[i].record(stream)
            run_one()
            ends[i].record(stream)
        torch.cuda.synchronize()
        return [s.elapsed_time(e) for s, e in zip(starts, ends)], time.perf_counter() - t0

    def kernel_times(g, step, n):
        # per-kernel durations: HIP events around each launch, on extra steps
        g.set_profiling(True)
        for _ in range(n):
            flush_caches()
            step()
        kt = g.kernel_times()
        g.set_profiling(False)
        torch.cuda.synchronize()
        return kt

    def make_handle(w, headline):
        opts = None
        if headline and (args.tile_cfg >= 0 or args.split > 0 or args.window > 0 or args.ring != "auto"):
            opts = pkg.options(tile_cfg=args.tile_cfg, split=args.split, chunks_per_window=args.window,
                               precision=prec, a_format=args.a_format, b_format=args.b_format,
                               ring=-1 if args.ring == "auto" else args.ring)
        elif prec != pkg.PRECISION_EXACT or fmts != ("e4m3", "e4m3"):
            opts = pkg.options(precision=prec, a_format=args.a_format, b_format=args.b_format)
        return pkg.SegGemm(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf, opts=opts)

    w = inputs.WORKLOADS[args.config]
    log(f"[bench] {args.config}: {w.describe()}")
    a_q, a_s, b_q, b_s, c = make_inputs(w)
    # identity of the run's inputs: SHA-256 of the quantised operands as they
    # sit in device memory (A codes, A scales, B codes, B scales, in order)
    hq = hashlib.sha256()
    for t in (a_q, a_s, b_q, b_s):
        hq.update(t.cpu().numpy().tobytes())
    inputs_sha = hq.hexdigest()[:16]
    props = torch.cuda.get_device_properties(dev)
    import numpy as _np
    env = {"device": props.name, "arch": getattr(props, "gcnArchName", None),
           "compute_units": props.multi_processor_count, "torch": torch.__version__,
           "hip": torch.version.hip, "numpy": _np.__version__}

    g = make_handle(w, True)
    plan = g.plan.as_dict()
    log(f"[bench] plan: {plan}")

    def step():
        g.run(a_q, a_s, b_q, b_s, c, stream=stream)

    # warm-up: the first call is discarded; before each timed loop, the
    # steps of that loop run untimed for at least --warmup steps and at
    # least --warmup-ms of GPU time (at most 200 steps), so the timed steps
    # do not start in the clock and power transient that follows an idle GPU
    flush_caches()
    step()
    torch.cuda.synchronize()
    warm_up(step, "stream")
    ms, wall = timed(step, args.steps)
    ms_mean = statistics.mean(ms)
    log(f"[bench] stream-issued: mean {ms_mean:.4f} ms median {statistics.median(ms):.4f} "
        f"min {min(ms):.4f} max {max(ms):.4f}")

    graph = None
    graph_ms = None
    if not args.no_graph:
        try:
            gs = torch.cuda.Stream()
            graph = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.stream(gs):
                with torch.cuda.graph(graph, stream=gs):
                    g.run(a_q, a_s, b_q, b_s, c, stream=gs)
            torch.cuda.synchronize()
        except Exception as e:  # report, time stream-issued steps only
            log(f"[bench] graph capture unavailable ({e})")
            graph = None
    if graph is not None:
        warm_up(graph.replay, "graph")
        gms, _ = timed(graph.replay, args.steps)
        graph_ms = statistics.mean(gms)
        log(f"[bench] graph replays: mean {graph_ms:.4f} ms")

    # ---- telemetry window: sustained steps while the sampler runs --------
    telemetry = None
    if sampler is not None:
        t0 = time.time()
        while time.time() - t0 < args.telemetry_seconds:
            for _ in range(8):
                if graph is not None:
                    graph.replay()
                else:
                    step()
            torch.cuda.synchronize()
        t1 = time.time()
        rows = read_samples(tele_path, t0, t1)
        if rows:
            mhz = [statistics.mean(r["gfx_mhz"]) for r in rows]
            telemetry = {"samples": len(rows), "shader_clock_mhz_median": round(statistics.median(mhz), 1),
                         "shader_clock_mhz_min": round(min(mhz), 1),
                         "socket_power_w_median": round(statistics.median(r["power_w"] for r in rows), 1),
                         "source": "amd-smi metric --clock --power (--temperature), mean over XCDs, "
                                   f"during {t1 - t0:.1f} s of back-to-back steps (no flush)"}
            for key, name in (("mem_mhz", "memory_clock_mhz_median"), ("temp_c", "temperature_c_median")):
                vals = [r[key] for r in rows if r.get(key) is not None]
                if vals:
                    telemetry[name] = round(statistics.median(vals), 1)
            log(f"[bench] telemetry: {telemetry}")
    if graph is not None:
        del graph

    kt = kernel_times(g, step, max(3, min(args.steps, 10)))
    gemm_ms_per_launch = kt["gemm_ms"] / kt["gemm_launches"]
    stage_ms_per_launch = kt["stage_ms"] / max(1, kt["stage_launches"])
    ring_flags = plan["ring"] == pkg.RING_FLAGS
    roof = gemm_roofline(w, plan, gemm_ms_per_launch, args.precision, ring_flags)
    log(f"[bench] kernels: gemm {gemm_ms_per_launch * 1e3:.2f} us/launch x{roof['launches_per_step']}, "
        f"stage {stage_ms_per_launch * 1e3:.2f} us/launch")

    sha = kernel_source_sha()
    traffic = load_traffic(args.config, args.precision, args.a_format, args.b_format,
                           "flags" if ring_flags else "events", plan, sha)
    roof["traffic"] = traffic
    roof["stage_us_per_launch"] = round(stage_ms_per_launch * 1e3, 3)
    roof["kernel"] = "GEMM kernel (" + ("bf16 MFMA, exact products" if args.precision == "exact"
                                        else "scaled FP8 MFMA") + ")"
    # the same fraction against the peak at the shader clock measured while
    # the kernel ran (MFMA bound only)
    roof["frac_at_measured_clock"] = (
        round(roof["achieved"] / (roof["peak"] * telemetry["shader_clock_mhz_median"] / 2400.0), 4)
        if telemetry and roof["bound"] == "mfma" else None)

    g.close()
    del a_q, a_s, b_q, b_s, c
    torch.cuda.empty_cache()

    # ---- the other workloads: stream timer, per-launch GEMM durations -----
    configs = {}
    if not args.no_configs:
        for name, wc in inputs.WORKLOADS.items():
            if name == args.config:
                continue
            log(f"[bench] workload {name}: {wc.describe()}")
            aq, as_, bq, bs, cc = make_inputs(wc)
            gc = make_handle(wc, False)
            pc = gc.plan.as_dict()

            def step_c():
                gc.run(aq, as_, bq, bs, cc, stream=stream)

            flush_caches()
            step_c()
            torch.cuda.synchronize()
            warm_up(step_c, name)
            cms, _ = timed(step_c, args.config_steps)
            # the second timer: the step captured once in a HIP graph, replayed
            gms_graph = None
            if not args.no_graph:
                try:
                    gsc = torch.cuda.Stream()
                    graph_c = torch.cuda.CUDAGraph()
                    torch.cuda.synchronize()
                    with torch.cuda.stream(gsc):
                        with torch.cuda.graph(graph_c, stream=gsc):
                            gc.run(aq, as_, bq, bs, cc, stream=gsc)
                    torch.cuda.synchronize()
                    warm_up(graph_c.replay, name + " graph")
                    gms_graph, _ = timed(graph_c.replay, args.config_steps)
                    del graph_c
                except Exception as e:  # report the stream timer only
                    log(f"[bench]   graph capture unavailable ({e})")
            ktc = kernel_times(gc, step_c, 5)
            gms_c = ktc["gemm_ms"] / ktc["gemm_launches"]
            rc = gemm_roofline(wc, pc, gms_c, args.precision, pc["ring"] == pkg.RING_FLAGS)
            med = statistics.median(cms)
            mean = statistics.mean(cms)
            configs[name] = {
                "shape": wc.describe(),
                "ms_per_step_mean": round(mean, 5), "ms_per_step_median": round(med, 5),
                "ms_per_step_min": round(min(cms), 5),
                "graph_ms_per_step_mean": round(statistics.mean(gms_graph), 5) if gms_graph else None,
                "tflops": round(wc.flops / (mean * 1e-3) / 1e12, 3),
                "pct_of_mxfp8_peak": round(100.0 * wc.flops / (mean * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 2),
                "hbm_frac_end_to_end": round(wc.algorithmic_bytes / (mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "gemm_us_per_launch": rc["gemm_us_per_launch"],
                "stage_us_per_launch": round(ktc["stage_ms"] / max(1, ktc["stage_launches"]) * 1e3, 3),
                "roofline": {k: rc[k] for k in ("bound", "achieved", "peak", "unit", "frac",
                                                "frac_of_kernel_mfma_peak", "frac_of_hbm",
                                                "launches_per_step")},
                "plan": {k: pc[k] for k in ("tile_m", "tile_n", "split", "chunks_per_window",
                                            "windows", "grid", "ring")},
            }
            log(f"[bench]   mean {mean:.4f} ms"
                + (f" (graph replays {statistics.mean(gms_graph):.4f} ms)" if gms_graph else "")
                + f", gemm {rc['gemm_us_per_launch']:.2f} us/launch, roofline {rc['bound']} {rc['frac']:.3f}")
            gc.close()
            del aq, as_, bq, bs, cc
            torch.cuda.empty_cache()

    peaks = None
    if not args.no_peaks:
        peaks = measured_peaks(torch, dev, stream)
        log(f"[bench] measured peaks: {peaks}")
        key = "bf16_mfma_tflops" if args.precision == "exact" else "scaled_fp8_mfma_tflops"
        if roof["bound"] == "mfma" and peaks.get("scaled_fp8_mfma_tflops"):
            roof["frac_of_measured_mxfp8_rate"] = round(roof["gemm_tflops"] / peaks["scaled_fp8_mfma_tflops"], 4)
            roof["frac_of_measured_kernel_mfma_rate"] = round(roof["gemm_tflops"] / peaks[key], 4)

    if sampler is not None:
        open(tele_path + ".stop", "w").close()
        try:
            sampler.wait(timeout=15)
        except Exception:
            sampler.kill()
        for f in (tele_path, tele_path + ".stop"):
            if os.path.exists(f):
                os.remove(f)

    value = float(w.flops) / (ms_mean * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_mean, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic the GEMM runs in: exact mode widens the FP8 codes
        # (scale folded in, exactly) to bfloat16 for the bf16 MFMA with FP32
        # accumulation; native mode multiplies the FP8 codes on the scaled
        # FP8 MFMA.  Inputs are MXFP8 either way.
        "dtype": "bf16" if args.precision == "exact" else "fp8",
        "inputs_dtype": f"mx{args.a_format}/mx{args.b_format} (E8M0 per 32), bf16 out",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {w.describe()}, "
                               f"N(0,{w.sigma:g})" + (f" with {w.outlier_frac:.0%} of entries "
                               f"x{w.outlier_mul:g}" if w.outlier_frac else "") +
                               f", seed {w.seed}; MXFP8 A {args.a_format.upper()}, "
                               f"B {args.b_format.upper()} + E8M0/32 in, bfloat16 out",
                   "flop_per_step": w.flops,
                   "algorithmic_bytes_per_step": w.algorithmic_bytes,
                   "plan": {k: plan[k] for k in ("tile_m", "tile_n", "split", "chunks_per_window",
                                                 "windows", "grid", "ring")}},
        "pct_of_mxfp8_peak": round(100.0 * value / PEAK_FP8_TFLOPS, 2),
        "hbm_frac_end_to_end": round(w.algorithmic_bytes / (ms_mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "timer": ("stream-issued steps, HIP events per step" + (", 512 MiB cache flush before each step"
                                                                  if not args.no_flush else ", warm caches")),
        "graph_ms_per_step": round(graph_ms, 5) if graph_ms is not None else None,
        "ms_per_step_median": round(statistics.median(ms), 5),
        "ms_per_step_min": round(min(ms), 5),
        "ms_per_step_p90": round(sorted(ms)[min(len(ms) - 1, int(0.9 * len(ms)))], 5),
        "telemetry": telemetry,
        "wall_s_timed_loop_incl_flush": round(wall, 4),
        "warmup_run": warm_log,
        "precision": args.precision,
        "roofline": roof,
        "configs": configs,
        "measured_peaks": peaks,
        "kernel_source_sha": sha,
        "inputs_sha256": inputs_sha,
        "env": env,
        # what "correct" means for this output (checked by the GPU tests
        # against the CPU oracle, not by the timed run)
        "acceptance": {
            "tolerance": "|gpu - oracle| <= 1e-2 + 8e-3 |oracle| elementwise, NaN fails; "
                         "quantiser codes and scales bit-exact",
            "pages_threshold": "the source's own check is allclose with rtol = atol = 1e-2 "
                               "on the bfloat16 output (context)",
        },
    }
    del flush
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a row sample")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
