"""GPU checks of the non-finite reading (the oracle header states it):
the quantiser's NaN and infinity blocks bit for bit against the oracle, and
the E8M0 NaN scale byte 0xFF in a GEMM input, which must turn exactly the
outputs its block feeds into NaN and leave every other output as it was."""
import numpy as np
import pytest

import oracle
from gpu_common import custom_case, say, summary, torch_cuda, within_tol

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_gpu_quantizer_nonfinite_blocks(fmt):
    torch = torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    rng = np.random.default_rng(21)
    x = rng.standard_normal((16, 256)).astype(np.float32)
    x[0, 3] = np.nan
    x[1, 40], x[1, 41] = np.inf, -np.inf
    x[2, 64], x[2, 65] = np.nan, np.inf
    x[3, 96:128] = np.nan
    x[4, 0:32] = -np.inf
    x[5, 32], x[5, 33] = np.float32(3.0e38), np.inf
    x[6, 160] = -np.nan
    x[7, 200] = np.float32(-0.0)
    x[7, 192:224] *= np.float32(2.0 ** -140)
    x[7, 201] = np.inf                                  # tiny values next to an infinity
    f = pkg.FMT_E4M3 if fmt == "e4m3" else pkg.FMT_E5M2
    q, s = pkg.quantize_mxfp8(torch.from_numpy(x).cuda(), fmt=f)
    qr, sr = oracle.quantize_mxfp8(x, fmt=fmt)
    say(f"[quant-nonfinite] {fmt}: scale bytes of the special blocks "
        f"{[int(sr[r, b]) for r, b in ((0, 0), (1, 1), (2, 2), (4, 0), (7, 6))]}")
    assert np.array_equal(s.cpu().numpy(), sr)
    assert np.array_equal(q.cpu().numpy(), qr)


def _run(case, opts, a_s=None, b_s=None):
    import torch
    import mxfp8_block_scaled_mxgemm_amd as pkg
    w = case.w
    c = torch.full((w.M, w.N), 7.0, dtype=torch.bfloat16, device="cuda:0")
    with pkg.SegGemm(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf, opts=opts) as g:
        g.run(case.a_q, case.a_s if a_s is None else a_s, case.b_q,
              case.b_s if b_s is None else b_s, c)
        torch.cuda.synchronize()
    return c.float().cpu().numpy()


@pytest.mark.parametrize("precision", ["exact", "native"])
@pytest.mark.parametrize("plan", ["large_tile", "small_tile_split", "flags"])
def test_gpu_nan_scale_byte(plan, precision):
    torch = torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    R, M, kpr, N, cms, nbuf = 4, 96, 256, 192, 16, 4
    case = custom_case(R=R, M=M, kpr=kpr, N=N, cms=cms, nbuf=nbuf, seed=31)
    prec = pkg.PRECISION_EXACT if precision == "exact" else pkg.PRECISION_NATIVE
    kw = {"large_tile": dict(tile_cfg=0 if precision == "native" else 1, split=1),
          "small_tile_split": dict(tile_cfg=5, split=2),
          "flags": dict(ring=pkg.RING_FLAGS)}[plan]
    opts = pkg.options(precision=prec, **kw)
    say(f"[nan-scale] {plan} {precision}")
    base = _run(case, opts)
    ref = case.oracle_full()
    bad, _ = within_tol(base, ref)
    assert not bad.any(), summary(base, ref)
    # A: segment 2, row 37, MX block 5 (K [2*256 + 160, +32)); B: row 101,
    # K block 3 of segment 1
    a_s = case.a_s.clone()
    a_s[2, 37, 5] = 0xFF
    b_s = case.b_s.clone()
    b_s[101, (1 * kpr) // 32 + 3] = 0xFF
    got = _run(case, opts, a_s=a_s, b_s=b_s)
    mask = np.zeros((M, N), bool)
    mask[37, :] = True
    mask[:, 101] = True
    say(f"  NaN outputs: {int(np.isnan(got).sum())} (expected {int(mask.sum())}); "
        f"non-NaN values there: {np.unique(got[mask & ~np.isnan(got)])[:6]}")
    assert np.all(np.isnan(got[mask]))
    assert np.array_equal(got[~mask], base[~mask])
