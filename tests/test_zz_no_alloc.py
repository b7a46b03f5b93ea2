"""The entry point that allocates nothing (mxgemm_seg_run_static), called
through the C ABI: its C must equal that of mxgemm_seg_run on a handle with
the same arguments (same plan, same kernels), on two calls in a row with the
second smaller -- whose split-K arrival counts sit where the first call left
partial sums, so they must be cleared -- and meet the oracle's tolerance."""
import ctypes

import numpy as np
import pytest

from gpu_common import custom_case, say, summary, torch_cuda, within_tol

pytestmark = pytest.mark.gpu


def _existing(case):
    import torch
    import mxfp8_block_scaled_mxgemm_amd as pkg
    w = case.w
    c = torch.full((w.M, w.N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    with pkg.SegGemm(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf) as g:
        g.run(case.a_q, case.a_s, case.b_q, case.b_s, c)
        torch.cuda.synchronize()
        plan = g.plan.as_dict()
    return c.float().cpu().numpy(), plan


def _static(case):
    import torch
    import mxfp8_block_scaled_mxgemm_amd as pkg
    w = case.w
    c = torch.full((w.M, w.N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    pkg.run_static(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf, case.a_q, case.a_s, case.b_q,
                   case.b_s, c)
    torch.cuda.synchronize()
    return c.float().cpu().numpy()


def test_static_entry_matches_the_handle_entry():
    torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    shapes = [(8, 64, 896, 2048, 8, 4, 104),     # skinny geometry: 16 x 64 tiles, fused split 8
              (4, 48, 512, 192, 16, 4, 7)]       # smaller, fused split 4
    for (R, M, kpr, N, cms, nbuf, seed) in shapes:
        say(f"[no-alloc] R={R} M={M} kpr={kpr} N={N} cms={cms} nbuf={nbuf}")
        case = custom_case(R=R, M=M, kpr=kpr, N=N, cms=cms, nbuf=nbuf, seed=seed)
        ref_c, plan = _existing(case)
        got = _static(case)
        sp = pkg.plan(M, kpr, R, N, cms, nbuf, opts=pkg.options(chunks_per_window=nbuf)).as_dict()
        same_plan = all(sp[k] == plan[k] for k in ("tile_cfg", "split", "chunks_per_window"))
        say(f"  plan {plan['tile_m']}x{plan['tile_n']} split {plan['split']} W {plan['chunks_per_window']}"
            f" (static: same plan {same_plan})")
        assert not np.isnan(got).any()
        if same_plan:
            assert np.array_equal(got, ref_c)
        ora = case.oracle_full()
        bad, _ = within_tol(got, ora)
        assert not bad.any(), summary(got, ora)


def test_static_entry_refuses_problems_beyond_its_scratch():
    torch = torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    lib = pkg.load()
    t = torch.zeros(64, dtype=torch.uint8, device="cuda:0")
    p = ctypes.c_void_p(t.data_ptr())
    # the 8192-cube workload with a ring of 8 buffers: 8 x 4 MiB + scales
    rc = lib.mxgemm_seg_run_static(8192, 1024, 8, 8192, 512, 8, None, p, p, p, p, p, None)
    assert rc == pkg._lib.MXGEMM_EUNSUPPORTED
    assert "static scratch" in pkg.last_error()
    o = pkg.options(ring=pkg.RING_FLAGS)
    rc = lib.mxgemm_seg_run_static(64, 256, 2, 64, 16, 2, ctypes.byref(o), p, p, p, p, p, None)
    assert rc == pkg._lib.MXGEMM_EUNSUPPORTED
