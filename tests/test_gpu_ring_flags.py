"""GPU tests of the device-flag ring protocol (one persistent launch per run):
parity with the oracle on the small workloads, chunk tails, every window
size, every format pair; counters reset between runs and under graph
replay; a run whose waits give up at once still ends and reports it."""
import numpy as np
import pytest

import oracle
from gpu_common import custom_case, say, summary, torch_cuda, within_tol, workload_case

pytestmark = pytest.mark.gpu

_CACHE = {}


def _flags(**kw):
    import mxfp8_block_scaled_mxgemm_amd as pkg
    return pkg.options(ring=pkg.RING_FLAGS, **kw)


def _run_checked(case, opts):
    """Run with the flags protocol, check the plan took it and no wait gave up."""
    import torch
    import mxfp8_block_scaled_mxgemm_amd as pkg
    w = case.w
    c = torch.full((w.M, w.N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    opts.a_format, opts.b_format = case.fmt_a, case.fmt_b
    with pkg.SegGemm(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf, opts=opts) as g:
        assert g.plan.ring == pkg.RING_FLAGS
        g.run(case.a_q, case.a_s, case.b_q, case.b_s, c)
        torch.cuda.synchronize()
        g.status()
    return c.float().cpu().numpy()


@pytest.mark.parametrize("name", ["tiny_m128_n256_k512", "skinny_m64_n2048_k7168",
                                  "m1024_n2048_k4096"])
def test_flags_parity_workloads(name):
    torch_cuda()
    say(f"[flags] {name}")
    case = workload_case(name)
    got = _run_checked(case, _flags())
    ref = case.oracle_full()
    say("  " + summary(got, ref))
    bad, _ = within_tol(got, ref)
    assert not bad.any()


@pytest.mark.parametrize("W", [1, 2, 4])
def test_flags_window_sizes(W):
    """Skinny geometry, every window size: one, two and four slot groups'
    worth of chunks per window (W = 4 leaves one slot group, so staging
    waits for the previous window's readers)."""
    torch_cuda()
    say(f"[flags-window] W={W}")
    if "skinny" not in _CACHE:
        _CACHE.clear()
        _CACHE["skinny"] = workload_case("skinny_m64_n2048_k7168")
        _CACHE["skinny_ref"] = _CACHE["skinny"].oracle_full()
    got = _run_checked(_CACHE["skinny"], _flags(chunks_per_window=W))
    bad, _ = within_tol(got, _CACHE["skinny_ref"])
    assert not bad.any(), summary(got, _CACHE["skinny_ref"])


@pytest.mark.parametrize("shape", [
    (4, 130, 256, 200, 48, 2),      # tail chunk, N not a multiple of 64 or 4
    (2, 1, 128, 64, 64, 4),         # a single one-row chunk
    (8, 70, 896, 2048, 8, 4),       # skinny with a 6-row last chunk
    (3, 1000, 384, 520, 96, 4),     # odd R, many tile rows per window
    (1, 96, 128, 64, 32, 1),        # one rank, one ring slot
    (2, 64, 512, 130, 16, 8),       # N = 130: ragged last tile column
])
def test_flags_ragged_shapes(shape):
    torch_cuda()
    R, M, kpr, N, cms, nbuf = shape
    say(f"[flags-ragged] R={R} M={M} kpr={kpr} N={N} cms={cms} nbuf={nbuf}")
    case = custom_case(R=R, M=M, kpr=kpr, N=N, cms=cms, nbuf=nbuf, seed=41 + M)
    got = _run_checked(case, _flags())
    ref = case.oracle_full()
    bad, _ = within_tol(got, ref)
    assert not bad.any(), summary(got, ref)


@pytest.mark.parametrize("fa,fb", [(oracle.E5M2, oracle.E5M2), (oracle.E4M3, oracle.E5M2),
                                   (oracle.E5M2, oracle.E4M3)])
def test_flags_formats(fa, fb):
    torch_cuda()
    say(f"[flags-fmt] fa={fa} fb={fb}")
    case = custom_case(R=8, M=64, kpr=896, N=512, cms=8, nbuf=4, seed=43, fmt_a=fa, fmt_b=fb)
    got = _run_checked(case, _flags())
    ref = case.oracle_full()
    bad, _ = within_tol(got, ref)
    assert not bad.any(), summary(got, ref)


@pytest.mark.parametrize("shape", [
    (8, 64, 896, 2048, 8, 4),       # skinny geometry
    (2, 128, 256, 256, 64, 2),      # tiny geometry
    (4, 130, 256, 200, 48, 2),      # tail chunk, ragged N
    (3, 1000, 384, 520, 96, 4),     # odd R, several tile rows per window
])
@pytest.mark.parametrize("fa,fb", [(oracle.E4M3, oracle.E4M3), (oracle.E5M2, oracle.E4M3)])
def test_flags_native_precision(shape, fa, fb):
    """The flags protocol on the scaled FP8 MFMA (native precision)."""
    torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    R, M, kpr, N, cms, nbuf = shape
    say(f"[flags-native] R={R} M={M} kpr={kpr} N={N} cms={cms} nbuf={nbuf} fa={fa} fb={fb}")
    case = custom_case(R=R, M=M, kpr=kpr, N=N, cms=cms, nbuf=nbuf, seed=47 + M, fmt_a=fa, fmt_b=fb)
    got = _run_checked(case, _flags(precision=pkg.PRECISION_NATIVE))
    ref = case.oracle_full()
    say("  " + summary(got, ref))
    bad, _ = within_tol(got, ref)
    assert not bad.any()


@pytest.mark.parametrize("precision", ["exact", "native"])
def test_flags_integer_data_bit_exact_both_precisions(precision):
    torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    from gpu_common import Case
    from mxfp8_block_scaled_mxgemm_amd import inputs
    R, M, kpr, N, cms, nbuf = 8, 64, 896, 1024, 8, 4
    w = inputs.Workload("sign", R, M, kpr, N, cms, nbuf, 1.0, 0.0, 1.0, 0)
    xa = inputs.sparse_sign_matrix((M, R * kpr), 0.03, 97)
    xb = inputs.sparse_sign_matrix((N, R * kpr), 0.03, 98)
    case = Case(w, xa, xb)
    ref = xa.astype(np.float64) @ xb.astype(np.float64).T
    prec = pkg.PRECISION_EXACT if precision == "exact" else pkg.PRECISION_NATIVE
    got = _run_checked(case, _flags(precision=prec))
    assert np.array_equal(got, ref.astype(np.float32))


def test_flags_integer_data_bit_exact():
    torch_cuda()
    from gpu_common import Case
    from mxfp8_block_scaled_mxgemm_amd import inputs
    R, M, kpr, N, cms, nbuf = 8, 64, 896, 2048, 8, 4
    w = inputs.Workload("sign", R, M, kpr, N, cms, nbuf, 1.0, 0.0, 1.0, 0)
    xa = inputs.sparse_sign_matrix((M, R * kpr), 0.03, 95)
    xb = inputs.sparse_sign_matrix((N, R * kpr), 0.03, 96)
    case = Case(w, xa, xb)
    ref = xa.astype(np.float64) @ xb.astype(np.float64).T
    got = _run_checked(case, _flags())
    assert np.array_equal(got, ref.astype(np.float32))


def test_flags_repeated_runs_and_graph_replay():
    """The counters go back to zero after every run: repeated eager runs
    and replays of a captured graph give identical C."""
    torch = torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    case = workload_case("skinny_m64_n2048_k7168")
    w = case.w
    ref = case.oracle_full()
    with pkg.SegGemm(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf, opts=_flags()) as g:
        outs = []
        for i in range(5):
            c = torch.full((w.M, w.N), float("nan"), dtype=torch.bfloat16, device="cuda")
            g.run(case.a_q, case.a_s, case.b_q, case.b_s, c)
            torch.cuda.synchronize()
            outs.append(c.float().cpu().numpy())
        for o in outs[1:]:
            assert np.array_equal(o, outs[0])
        bad, _ = within_tol(outs[0], ref)
        assert not bad.any()
        stream = torch.cuda.Stream()
        c = torch.zeros((w.M, w.N), dtype=torch.bfloat16, device="cuda")
        with torch.cuda.stream(stream):
            g.run(case.a_q, case.a_s, case.b_q, case.b_s, c, stream=stream)   # warm
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            g.run(case.a_q, case.a_s, case.b_q, case.b_s, c, stream=stream)
        for i in range(4):
            c.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(c.float().cpu().numpy(), outs[0]), f"replay {i}"
            # eager work between replays
            g.run(case.a_q, case.a_s, case.b_q, case.b_s, c)
            torch.cuda.synchronize()
        g.status()


def test_flags_waits_that_give_up_still_end():
    """spin_limit = 0: a wait that does not find its count at once gives
    up.  The launch still ends (every wave reaches the end), the handle
    reports it or the result is right, and the counters are back at zero
    for a handle with normal waits afterwards."""
    torch = torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    case = workload_case("skinny_m64_n2048_k7168")
    w = case.w
    ref = case.oracle_full()
    c = torch.full((w.M, w.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pkg.SegGemm(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf,
                     opts=_flags(spin_limit=0)) as g:
        for _ in range(3):
            g.run(case.a_q, case.a_s, case.b_q, case.b_s, c)
        torch.cuda.synchronize()
        try:
            g.status()
            gave_up = False
        except pkg.MxgemmError as e:
            assert "ETIMEOUT" in str(e)
            gave_up = True
        if not gave_up:
            bad, _ = within_tol(c.float().cpu().numpy(), ref)
            assert not bad.any()
        g.status()          # the mark was cleared
        # the same handle with its counters reset: run once more, it must
        # end again (result not checked: its waits still give up early)
        g.run(case.a_q, case.a_s, case.b_q, case.b_s, c)
        torch.cuda.synchronize()
    say(f"  waits gave up: {gave_up}")
    got = _run_checked(case, _flags())
    bad, _ = within_tol(got, ref)
    assert not bad.any()


def test_flags_profiling_counts_one_launch():
    torch = torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    case = custom_case(R=2, M=128, kpr=256, N=256, cms=64, nbuf=2, seed=45)
    w = case.w
    c = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    with pkg.SegGemm(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf, opts=_flags()) as g:
        g.set_profiling(True)
        for _ in range(3):
            g.run(case.a_q, case.a_s, case.b_q, case.b_s, c)
        kt = g.kernel_times()
        g.set_profiling(False)
    assert kt["gemm_launches"] == 3 and kt["stage_launches"] == 0
    assert kt["gemm_ms"] > 0
