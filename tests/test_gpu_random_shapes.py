"""Parity on seeded random shapes (rank count, rows, K per rank, N, chunk
rows not dividing M, ring depth): every output of C against the oracle, in
exact mode with the automatic plan and with one forced tile configuration
the shape admits, and in native mode with the automatic plan.  A third of
the shapes carry 1% outliers x100 (exact mode only: the native MFMA's
in-group truncation is characterised elsewhere)."""
import numpy as np
import pytest

from gpu_common import (Case, K_GROUP_CFG, K_GROUPS, ONE_SHOT_CFG, ONE_SHOT_STEPS, say, summary,
                        torch_cuda, within_tol)
from random_shapes import random_shapes
from mxfp8_block_scaled_mxgemm_amd import inputs

pytestmark = pytest.mark.gpu

SHAPES = random_shapes(77, 24)


def _forced(i, R, kpr):
    """A tile configuration and split the shape admits, chosen by index."""
    rng = np.random.default_rng(1000 + i)
    for _ in range(100):
        cfg = int(rng.choice([1, 2, 3, 4, 5, 6, 7]))
        splits = [s for s in range(1, R + 1) if R % s == 0]
        s = int(rng.choice(splits))
        steps = (R // s) * (kpr // 128)
        if cfg == ONE_SHOT_CFG and steps > ONE_SHOT_STEPS:
            continue
        if cfg == K_GROUP_CFG and steps % K_GROUPS != 0:
            continue
        return cfg, s
    return 3, 1


@pytest.mark.parametrize("i", range(len(SHAPES)))
def test_parity_random_shape(i):
    torch_cuda()
    import mxfp8_block_scaled_mxgemm_amd as pkg
    R, M, kpr, N, cms, nbuf = SHAPES[i]
    outliers = i % 3 == 2
    w = inputs.Workload("random", R, M, kpr, N, cms, nbuf, 1.0, 0.01 if outliers else 0.0,
                        100.0 if outliers else 1.0, 5000 + i)
    a32, b32 = inputs.fp32_operands(w)
    case = Case(w, a32, b32)
    ref = case.oracle_full()
    cfg, split = _forced(i, R, kpr)
    runs = [("exact auto", pkg.options()),
            (f"exact cfg {cfg} split {split}", pkg.options(tile_cfg=cfg, split=split))]
    if not outliers:
        runs.append(("native auto", pkg.options(precision=pkg.PRECISION_NATIVE)))
    for label, opts in runs:
        say(f"[random {i}] R={R} M={M} kpr={kpr} N={N} cms={cms} nbuf={nbuf} outliers={outliers}: {label}")
        got = case.run_gpu(opts=opts).float().cpu().numpy()
        bad, _ = within_tol(got, ref)
        assert not bad.any(), summary(got, ref)
