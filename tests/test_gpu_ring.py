"""GPU behaviour of the staging ring and the C ABI: repeated and concurrent
runs, graph capture and replay, full overwrite of C, argument errors and
the measurement hooks."""
import ctypes

import numpy as np
import pytest

from gpu_common import custom_case, say, summary, torch_cuda, within_tol

pytestmark = pytest.mark.gpu

_CASE = {}


def _case():
    if "c" not in _CASE:
        # 16 chunks through a 4-deep ring: every slot is refilled 3 times
        _CASE["c"] = custom_case(R=4, M=512, kpr=512, N=512, cms=32, nbuf=4, seed=91)
    return _CASE["c"]


def test_repeated_runs_identical_and_correct():
    torch = torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    case = _case()
    w = case.w
    ref = case.oracle_full()
    for label, opts in (("auto", None), ("64x64 split 4", pkg.options(split=4, tile_cfg=3)),
                        ("256x128", pkg.options(split=1, tile_cfg=1)),
                        ("64x64 K groups", pkg.options(split=1, tile_cfg=7))):
        say(f"[repeat] opts={label}")
        outs = []
        with pkg.SegGemm(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf, opts=opts) as g:
            for _ in range(5):
                c = torch.full((w.M, w.N), float("nan"), dtype=torch.bfloat16, device="cuda")
                g.run(case.a_q, case.a_s, case.b_q, case.b_s, c)
                outs.append(c)
            torch.cuda.synchronize()
        first = outs[0].float().cpu().numpy()
        bad, _ = within_tol(first, ref)
        assert not bad.any(), summary(first, ref)
        for o in outs[1:]:
            assert np.array_equal(o.float().cpu().numpy(), first)   # deterministic


@pytest.mark.parametrize("tiles", ["auto split 2", "256x128", "64x64 K groups"])
def test_graph_capture_replays(tiles):
    torch = torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    case = _case()
    w = case.w
    opts = {"auto split 2": pkg.options(split=2), "256x128": pkg.options(split=1, tile_cfg=1),
            "64x64 K groups": pkg.options(split=1, tile_cfg=7)}[tiles]
    say(f"[graph] {tiles}: capture + 4 replays")
    with pkg.SegGemm(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf, opts=opts) as g:
        eager = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
        g.run(case.a_q, case.a_s, case.b_q, case.b_s, eager)
        torch.cuda.synchronize()
        c = torch.empty_like(eager)
        s = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                g.run(case.a_q, case.a_s, case.b_q, case.b_s, c, stream=s)
        torch.cuda.synchronize()
        for i in range(4):
            c.fill_(float("nan"))
            junk = torch.randn(1 << 20, device="cuda") * 2        # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(c, eager), f"replay {i}"
            del junk
        # eager runs still work after the capture
        c2 = torch.empty_like(eager)
        g.run(case.a_q, case.a_s, case.b_q, case.b_s, c2)
        torch.cuda.synchronize()
        assert torch.equal(c2, eager)


def test_two_handles_two_streams():
    torch = torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    case = _case()
    w = case.w
    other = custom_case(R=2, M=256, kpr=256, N=320, cms=64, nbuf=2, seed=92)
    wo = other.w
    say("[streams] two handles concurrently")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    g1 = pkg.SegGemm(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf)
    g2 = pkg.SegGemm(wo.M, wo.kPerRank, wo.R, wo.N, wo.commMSize, wo.nbuf)
    c1 = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    c2 = torch.empty((wo.M, wo.N), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        g1.run(case.a_q, case.a_s, case.b_q, case.b_s, c1, stream=s1)
        g2.run(other.a_q, other.a_s, other.b_q, other.b_s, c2, stream=s2)
    torch.cuda.synchronize()
    g1.close()
    g2.close()
    for got, cs in ((c1, case), (c2, other)):
        got = got.float().cpu().numpy()
        bad, _ = within_tol(got, cs.oracle_full())
        assert not bad.any()


def test_argument_errors_on_device():
    torch = torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    from mxfp8_block_scaled_mxgemm_amd import _lib
    case = _case()
    w = case.w
    c = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    with pkg.SegGemm(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf) as g:
        lib = _lib.load()
        ptrs = [case.a_q.data_ptr(), case.a_s.data_ptr(), case.b_q.data_ptr(),
                case.b_s.data_ptr(), c.data_ptr()]
        for i in range(5):
            bad = list(ptrs)
            bad[i] = 0
            rc = lib.mxgemm_seg_run(g._h, *[ctypes.c_void_p(x) for x in bad], None)
            assert rc == _lib.MXGEMM_EINVAL
        bad = list(ptrs)
        bad[0] += 1                                      # misaligned A
        rc = lib.mxgemm_seg_run(g._h, *[ctypes.c_void_p(x) for x in bad], None)
        assert rc == _lib.MXGEMM_EINVAL
        with pytest.raises(ValueError):
            g.run(case.a_q[:, :-1], case.a_s, case.b_q, case.b_s, c)
    assert lib.mxgemm_seg_run(None, *[ctypes.c_void_p(x) for x in ptrs], None) == _lib.MXGEMM_EINVAL
    assert lib.mxgemm_seg_destroy(None) == 0


def test_profiling_counts_launches():
    torch = torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    case = _case()
    w = case.w
    with pkg.SegGemm(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf) as g:
        p = g.plan
        c = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
        g.set_profiling(True)
        for _ in range(3):
            g.run(case.a_q, case.a_s, case.b_q, case.b_s, c)
        t = g.kernel_times()
        g.set_profiling(False)
        assert t["gemm_launches"] == 3 * p.windows and t["stage_launches"] == 3 * p.windows
        assert t["gemm_ms"] > 0 and t["stage_ms"] > 0
        bad, _ = within_tol(c.float().cpu().numpy(), case.oracle_full())
        assert not bad.any()


def test_allocation_failure_is_enomem_and_leaves_no_error_behind():
    """create() with a split-K workspace far beyond device memory (8 splits
    x 65536 rows x 2^20 columns x 4 bytes = 2 TiB) fails with ENOMEM, frees
    what it had allocated, and leaves no HIP error that a later handle's
    launch checks would pick up."""
    torch = torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    from mxfp8_block_scaled_mxgemm_amd import _lib
    say("[enomem] 2 TiB workspace request")
    with pytest.raises(pkg.MxgemmError) as ei:
        pkg.SegGemm(65536, 128, 8, 1 << 20, 65536, 1, opts=pkg.options(tile_cfg=1, split=8))
    assert ei.value.code == _lib.MXGEMM_ENOMEM
    case = _case()
    got = case.run_gpu().float().cpu().numpy()
    torch.cuda.synchronize()
    bad, _ = within_tol(got, case.oracle_full())
    assert not bad.any()


def test_run_refuses_host_memory_the_gpu_cannot_use():
    """run() checks its buffers before enqueuing anything: pageable host
    memory in any argument is refused with EINVAL, and a correct call right
    after still runs."""
    torch = torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    from mxfp8_block_scaled_mxgemm_amd import _lib
    case = _case()
    w = case.w
    c = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    host = np.zeros(w.M * w.N * 2 + 64, dtype=np.uint8)         # pageable host memory
    host_ptr = (host.ctypes.data + 15) // 16 * 16
    lib = _lib.load()
    ptrs = [case.a_q.data_ptr(), case.a_s.data_ptr(), case.b_q.data_ptr(), case.b_s.data_ptr(),
            c.data_ptr()]
    with pkg.SegGemm(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf) as g:
        for i in range(5):
            bad = list(ptrs)
            bad[i] = host_ptr
            say(f"[buffers] host pointer in argument {i}")
            rc = lib.mxgemm_seg_run(g._h, *[ctypes.c_void_p(x) for x in bad], None)
            assert rc == _lib.MXGEMM_EINVAL, lib.mxgemm_seg_last_error()
            assert b"not memory the GPU can access" in lib.mxgemm_seg_last_error()
        torch.cuda.synchronize()
        c.fill_(float("nan"))
        g.run(case.a_q, case.a_s, case.b_q, case.b_s, c)
        torch.cuda.synchronize()
    got = c.float().cpu().numpy()
    bad, _ = within_tol(got, case.oracle_full())
    assert not bad.any()


def test_quantizer_refuses_host_memory():
    """The quantiser's C entry refuses pageable host memory for its input
    and outputs before launching, and works on device memory right after."""
    torch = torch_cuda()
    from mxfp8_block_scaled_mxgemm_amd import _lib
    lib = _lib.load()
    rows, cols = 8, 64
    x = torch.randn((rows, cols), device="cuda")
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    host = np.zeros(rows * cols * 4 + 64, dtype=np.uint8)
    hp = (host.ctypes.data + 15) // 16 * 16
    dev = [x.data_ptr(), q.data_ptr(), s.data_ptr()]
    for i in range(3):
        args = list(dev)
        args[i] = hp
        say(f"[quantiser] host pointer in argument {i}")
        rc = lib.mxgemm_quantize_mx(ctypes.c_void_p(args[0]), rows, cols, cols, ctypes.c_void_p(args[1]),
                                    cols, ctypes.c_void_p(args[2]), cols // 32, 0, None)
        assert rc == _lib.MXGEMM_EINVAL
        assert b"not memory the GPU can access" in lib.mxgemm_seg_last_error()
    rc = lib.mxgemm_quantize_mx(ctypes.c_void_p(dev[0]), rows, cols, cols, ctypes.c_void_p(dev[1]), cols,
                                ctypes.c_void_p(dev[2]), cols // 32, 0, None)
    assert rc == _lib.MXGEMM_OK
    torch.cuda.synchronize()
    assert int(s.max()) > 0
