"""Shared helpers for the GPU tests (imported by test modules, not collected)."""
import sys

import numpy as np
import pytest

import oracle
from mxfp8_block_scaled_mxgemm_amd import inputs

# Acceptance rule: |gpu - oracle| <= ATOL + RTOL * |oracle|, NaN fails.
# (The pages' own check is torch.allclose with rtol = atol = 1e-2 on bfloat16
# outputs; this rule is tighter in the relative term.)
ATOL = 1e-2
RTOL = 8e-3


# The tile table as the tests see it (index = tile_cfg option).
NUM_TILE_CFGS = 8
NATIVE_ONLY_CFG = 0          # 256 x 256: no exact-mode kernel
ONE_SHOT_CFG, ONE_SHOT_STEPS = 6, 8
K_GROUP_CFG, K_GROUPS = 7, 4  # 64 x 64 in four K groups


def forced_tile_refused(cfg, split, R, kpr, precision):
    """True where forcing (cfg, split) must fail with MxgemmError: a
    one-shot work item longer than its single stage, a tile without a kernel
    for the precision mode, or K groups that cannot share the work item's
    K-steps evenly."""
    steps = (R // split) * (kpr // 128)
    if cfg == ONE_SHOT_CFG and steps > ONE_SHOT_STEPS:
        return True
    if cfg == NATIVE_ONLY_CFG and precision == "exact":
        return True
    if cfg == K_GROUP_CFG and steps % K_GROUPS != 0:
        return True
    return False


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def within_tol(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    bad = ~(d <= ATOL + RTOL * np.abs(ref))       # NaN compares False -> bad
    return bad, d


def report_misses(got, ref, ms=None, ns=None, limit=12):
    """Print the entries over tolerance (index, oracle value, GPU value,
    difference), largest excess first."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bad, d = within_tol(got, ref)
    idx = np.flatnonzero(bad)
    if idx.size == 0:
        return
    excess = d[idx] - (ATOL + RTOL * np.abs(ref[idx]))
    for i in idx[np.argsort(-excess)][:limit]:
        where = f"({int(ms[i])},{int(ns[i])})" if ms is not None else f"[{int(i)}]"
        say(f"    miss {where}: oracle {ref[i]:.6g} gpu {got[i]:.6g} |d| {d[i]:.4g} "
            f"tol {ATOL + RTOL * abs(ref[i]):.4g}")


def summary(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bad, d = within_tol(got, ref)
    rel = d / np.maximum(np.abs(ref), 1e-8)
    return (f"n={got.size} max_abs={np.nanmax(d):.3e} mean_abs={np.nanmean(d):.3e} "
            f"rmse={np.sqrt(np.nanmean(d * d)):.3e} max_rel={np.nanmax(rel):.3e} "
            f"over_tol={int(bad.sum())} identical={np.mean(got == ref):.4f}")


class Case:
    """One workload: fp32 operands, the GPU-quantised device tensors and the
    oracle-quantised host arrays; A codes of format fmt_a, B codes of fmt_b
    (oracle.E4M3 / oracle.E5M2, the same codes as the library's)."""

    def __init__(self, w, a32, b32, fmt_a=oracle.E4M3, fmt_b=oracle.E4M3):
        import torch
        import mxfp8_block_scaled_mxgemm_amd as pkg
        self.w = w
        self.fmt_a, self.fmt_b = fmt_a, fmt_b
        dev = torch.device("cuda:0")
        self.a32, self.b32 = a32, b32
        a_d = torch.from_numpy(a32).to(dev)
        b_d = torch.from_numpy(b32).to(dev)
        self.a_q, self.a_s = pkg.quantize_segments(a_d, w.R, fmt=fmt_a)
        self.b_q, self.b_s = pkg.quantize_mxfp8(b_d, fmt=fmt_b)
        del a_d, b_d
        qa, sa = oracle.quantize_mxfp8(a32, fmt=fmt_a)
        self.qb, self.sb = oracle.quantize_mxfp8(b32, fmt=fmt_b)
        self.a_seg = inputs.split_segments(qa, w.R)
        self.s_seg = inputs.split_segments(sa, w.R)
        torch.cuda.synchronize()

    def quantizer_matches(self):
        return (np.array_equal(self.a_q.cpu().numpy(), self.a_seg)
                and np.array_equal(self.a_s.cpu().numpy(), self.s_seg)
                and np.array_equal(self.b_q.cpu().numpy(), self.qb)
                and np.array_equal(self.b_s.cpu().numpy(), self.sb))

    def run_gpu(self, opts=None, c=None):
        import torch
        import mxfp8_block_scaled_mxgemm_amd as pkg
        w = self.w
        if c is None:
            c = torch.full((w.M, w.N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        if opts is None:
            opts = pkg.options()
        opts.a_format, opts.b_format = self.fmt_a, self.fmt_b
        with pkg.SegGemm(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf, opts=opts) as g:
            g.run(self.a_q, self.a_s, self.b_q, self.b_s, c)
            torch.cuda.synchronize()
        return c

    def oracle_full(self):
        return oracle.bf16_bits_to_float(
            oracle.mxgemm_seg(self.a_seg, self.s_seg, self.qb, self.sb, fmt_a=self.fmt_a,
                              fmt_b=self.fmt_b)).astype(np.float64)

    def oracle_entries(self, ms, ns):
        return oracle.bf16_bits_to_float(
            oracle.mxgemm_seg_entries(self.a_seg, self.s_seg, self.qb, self.sb, ms, ns,
                                      fmt_a=self.fmt_a, fmt_b=self.fmt_b)).astype(np.float64)


def workload_case(name, fmt_a=oracle.E4M3, fmt_b=oracle.E4M3):
    w = inputs.WORKLOADS[name]
    a32, b32 = inputs.fp32_operands(w)
    return Case(w, a32, b32, fmt_a, fmt_b)


def custom_case(R, M, kpr, N, cms, nbuf, seed, sigma=1.0, fmt_a=oracle.E4M3, fmt_b=oracle.E4M3):
    w = inputs.Workload("custom", R, M, kpr, N, cms, nbuf, sigma, 0.0, 1.0, seed)
    a32, b32 = inputs.fp32_operands(w)
    return Case(w, a32, b32, fmt_a, fmt_b)


def sample_entries(M, N, tile_m, tile_n, seed, count=4096):
    """Random entries plus every row/column on both sides of each tile edge
    (sampled along the other axis)."""
    rng = np.random.default_rng(seed)
    ms = list(rng.integers(0, M, count))
    ns = list(rng.integers(0, N, count))
    edge_m = sorted({x for t in range(0, M + 1, tile_m) for x in (t - 1, t) if 0 <= x < M})
    edge_n = sorted({x for t in range(0, N + 1, tile_n) for x in (t - 1, t) if 0 <= x < N})
    for m in edge_m[:64]:
        cols = rng.integers(0, N, 8)
        ms += [m] * len(cols)
        ns += list(cols)
    for n in edge_n[:64]:
        rows = rng.integers(0, M, 8)
        ns += [n] * len(rows)
        ms += list(rows)
    return np.array(ms, dtype=np.int64), np.array(ns, dtype=np.int64)


def tail_and_random_entries(got_all, seed, frac=0.05, count=1 << 20):
    """Entries to check on a large output: every output whose |C| (as the GPU
    computed it) is below ``frac`` times the RMS of C -- where the absolute
    term of the tolerance is all the budget there is -- plus ``count``
    uniformly random entries."""
    g = np.asarray(got_all)
    rms = float(np.sqrt(np.mean(np.square(g, dtype=np.float64))))
    tail = np.flatnonzero(np.abs(g) < frac * rms)
    rng = np.random.default_rng(seed)
    rand = rng.integers(0, g.size, count)
    flat = np.unique(np.concatenate([tail, rand]))
    ms, ns = np.divmod(flat, g.shape[1])
    return ms.astype(np.int64), ns.astype(np.int64), rms, tail.size
