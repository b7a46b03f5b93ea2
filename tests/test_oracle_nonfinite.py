"""Pins for the oracle's reading of non-finite inputs and of the E8M0 NaN
scale byte (the pages' generator is not shown, so the reading is ours; it is
written in the oracle's header):

* a block holding a NaN: scale byte 0xFF (E8M0 NaN), every code 0x7F;
* a block holding an infinity and no NaN: e = 127 (the clamp of +inf),
  infinities saturate to the largest finite code of their sign, finite
  elements encode as x * 2^-127;
* a scale byte 0xFF in a GEMM input makes every output that takes a product
  from its block NaN and leaves every other output unchanged.

Codes of finite elements are checked against torch's float8 casts (a library
routine); the rest against the closed forms above.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_mxgemm_amd import inputs

INF, NAN = float("inf"), float("nan")

# format -> (largest finite code, torch dtype, E8M0 exponent function)
FMTS = {
    "e4m3": (0x7E, torch.float8_e4m3fn, oracle.e8m0_exponent),
    "e5m2": (0x7B, torch.float8_e5m2, oracle.e8m0_exponent_e5m2),
}


def _encode(fmt, v):
    return (oracle.e4m3_encode if fmt == "e4m3" else oracle.e5m2_encode)(np.asarray(v, np.float64))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_encode_nonfinite(fmt):
    top = FMTS[fmt][0]
    got = _encode(fmt, [INF, -INF, NAN, -NAN])
    assert got.tolist() == [top, 0x80 | top, 0x7F, 0x7F]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_e8m0_exponent_nonfinite(fmt):
    fn = FMTS[fmt][2]
    got = fn(np.array([INF, NAN, 0.0, 3.0e38]))
    assert got[0] == 127 and got[1] == 128 and got[2] == -127
    # the largest float32 magnitudes still get their own finite exponent
    fmax = 448.0 if fmt == "e4m3" else 57344.0
    assert fmax * 2.0 ** got[3] >= 3.0e38 > fmax * 2.0 ** (got[3] - 1)


def _torch_codes(y, dt):
    return torch.from_numpy(np.asarray(y, np.float32).copy()).to(dt).view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantizer_nonfinite_blocks(fmt):
    top, dt, _ = FMTS[fmt]
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 128)).astype(np.float32)
    x[0, 3] = np.nan                                   # NaN block
    x[1, 40] = np.inf                                  # +inf block
    x[1, 41] = -np.inf
    x[2, 64] = np.nan                                  # NaN beats inf in one block
    x[2, 65] = np.inf
    x[3, 96:128] = np.nan                              # all NaN
    x[4, 0:32] = -np.inf                               # all -inf
    x[5, 32] = np.float32(3.0e38)                      # a huge finite next to an inf
    x[5, 33] = np.inf
    q, s = oracle.quantize_mxfp8(x, fmt=fmt)
    # NaN blocks
    for (r, b) in ((0, 0), (2, 2), (3, 3)):
        assert s[r, b] == 0xFF
        assert np.all(q[r, 32 * b:32 * b + 32] == 0x7F)
    # infinity blocks: e = 127
    for (r, b) in ((1, 1), (4, 0), (5, 1)):
        assert s[r, b] == 254
        blk = x[r, 32 * b:32 * b + 32].astype(np.float64)
        exp = np.where(np.isposinf(blk), top, np.where(np.isneginf(blk), 0x80 | top, 0))
        fin = np.isfinite(blk)
        exp[fin] = _torch_codes(blk[fin] * 2.0 ** -127, dt)
        assert np.array_equal(q[r, 32 * b:32 * b + 32], exp.astype(np.uint8))
    # 3e38 * 2^-127 = 1.76..: an ordinary normal code
    assert q[5, 32] == _torch_codes([3.0e38 * 2.0 ** -127], dt)[0]
    # every other block is the finite rule (torch path)
    finite_blocks = [(r, b) for r in range(6) for b in range(4)
                     if np.all(np.isfinite(x[r, 32 * b:32 * b + 32]))]
    assert len(finite_blocks) == 18
    for (r, b) in finite_blocks:
        blk = x[r, 32 * b:32 * b + 32].astype(np.float64)
        amax = np.abs(blk).max()
        e = -127
        fmax = 448.0 if fmt == "e4m3" else 57344.0
        while fmax * 2.0 ** e < amax:
            e += 1
        assert s[r, b] == e + 127
        assert np.array_equal(q[r, 32 * b:32 * b + 32], _torch_codes(blk * 2.0 ** -e, dt))


@pytest.mark.parametrize("operand", ["A", "B"])
def test_gemm_nan_scale_byte(operand):
    """A scale byte 0xFF: the outputs its block feeds are NaN (NaN times
    any value, zero included, is NaN), every other output is unchanged."""
    R, M, kpr, N = 2, 12, 64, 10
    a = inputs.random_codes((R, M, kpr), 3, choices=[c for c in range(256) if c & 0x7F != 0x7F])
    b = inputs.random_codes((N, R * kpr), 4, choices=[c for c in range(256) if c & 0x7F != 0x7F])
    sa = inputs.random_scale_bytes((R, M, kpr // 32), 5, 120, 130)
    sb = inputs.random_scale_bytes((N, R * kpr // 32), 6, 120, 130)
    base = oracle.bf16_bits_to_float(oracle.mxgemm_seg(a, sa, b, sb))
    assert np.all(np.isfinite(base))
    a[1, 4, 7] = 0                         # a zero code inside the NaN block: still NaN
    base = oracle.bf16_bits_to_float(oracle.mxgemm_seg(a, sa, b, sb))
    if operand == "A":
        sa[1, 4, 0] = 0xFF                 # segment 1, row 4, K [64, 96)
    else:
        sb[7, 3] = 0xFF                    # column 7, K [96, 128)
    got = oracle.bf16_bits_to_float(oracle.mxgemm_seg(a, sa, b, sb))
    mask = np.zeros((M, N), bool)
    if operand == "A":
        mask[4, :] = True
    else:
        mask[:, 7] = True
    assert np.all(np.isnan(got[mask]))
    assert np.array_equal(got[~mask], base[~mask])
