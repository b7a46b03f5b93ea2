"""Pins for the oracle's second FP8 operand format, E5M2 (the sibling kernel
entries E5M2E5M2, E4M3E5M2 and E5M2E4M3 of all_to_all_matmul_impl.h):
decode and encode against torch's float8_e5m2 and the OCP spec points, the
E8M0 rule for the E5M2 largest finite 57344 by exact-rational brute force,
the quantiser against an independent torch path, and the mixed-format GEMM
against exact rational sums and numpy's float64 product.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_mxgemm_amd import inputs
from test_oracle_gemm import _bf16_rne_fraction, _near_midpoint

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E5M2_MAX = 57344.0
FINITE_E5M2 = [c for c in range(256) if (c & 0x7C) != 0x7C]
FINITE_E4M3 = [c for c in range(256) if c not in (0x7F, 0xFF)]


def _torch_value(codes, fmt):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy())
    dt = torch.float8_e5m2 if fmt == oracle.E5M2 else torch.float8_e4m3fn
    return t.view(dt).to(torch.float64).numpy()


def _torch_e5m2_encode(f32):
    t = torch.from_numpy(np.asarray(f32, dtype=np.float32).copy())
    return t.to(torch.float8_e5m2).view(torch.uint8).numpy()


def test_e5m2_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e5m2_value(codes)
    ref = _torch_value(codes, oracle.E5M2)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert set(np.nonzero(np.isnan(ours))[0].tolist()) == {0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF}
    ok = ~np.isnan(ours)
    assert np.array_equal(ours[ok], ref[ok])
    assert ours[0x7C] == math.inf and ours[0xFC] == -math.inf
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e5m2_decode_spec_points():
    with open(os.path.join(GOLDEN, "e5m2_spec_points.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            code, val = line.split()
            got = float(oracle.e5m2_value([int(code, 16)])[0])
            if val == "nan":
                assert math.isnan(got), code
            else:
                assert got == float(val), code
                assert math.copysign(1.0, got) == math.copysign(1.0, float(val))


def _structured_fp32():
    lows = np.array([0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x3FFF, 0x7FFF,
                     0x8000, 0xFFFF, 0x12345], dtype=np.uint32) & np.uint32(0x1FFFF)
    exps = np.arange(0, 143, dtype=np.uint32)          # biased; 142 -> [32768, 65536)
    top = np.arange(64, dtype=np.uint32)               # mantissa bits 22..17
    sign = np.array([0, 1], dtype=np.uint32)
    g = np.meshgrid(sign, exps, top, lows, indexing="ij")
    bits = (g[0] << 31) | (g[1] << 23) | (g[2] << 17) | g[3]
    f = bits.ravel().view(np.float32)
    return f[np.abs(f) <= np.float32(E5M2_MAX)]


def test_e5m2_encode_matches_torch_structured():
    f = _structured_fp32()
    ours = oracle.e5m2_encode(f.astype(np.float64))
    ref = _torch_e5m2_encode(f)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(float(f[i]), hex(ours[i]), hex(ref[i])) for i in bad[:10]]


def test_e5m2_encode_matches_torch_random():
    rng = np.random.default_rng(17)
    f = rng.integers(0, 2**32, size=1 << 22, dtype=np.uint64).astype(np.uint32).view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) <= np.float32(E5M2_MAX))]
    assert np.array_equal(oracle.e5m2_encode(f.astype(np.float64)), _torch_e5m2_encode(f))


def test_e5m2_encode_exhaustive_matches_torch():
    """All 2 x 1.19e9 fp32 values with |v| <= 57344 (0x47600000), in
    chunks, against torch's cast."""
    chunk = 1 << 26
    for sign in (0, 0x80000000):
        for lo in range(0, 0x47600000 + 1, chunk):
            hi = min(lo + chunk, 0x47600000 + 1)
            bits = np.arange(lo, hi, dtype=np.uint32) | np.uint32(sign)
            f = bits.view(np.float32)
            ref = torch.from_numpy(f).to(torch.float8_e5m2).view(torch.uint8).numpy()
            ours = oracle.e5m2_encode(f.astype(np.float64))
            if not np.array_equal(ours, ref):
                i = int(np.nonzero(ours != ref)[0][0])
                raise AssertionError(f"{float(f[i])!r}: oracle {int(ours[i]):#04x}, torch {int(ref[i]):#04x}")


def test_e5m2_encode_saturates_and_keeps_nan():
    big = np.array([57344.0, 61439.99, 61440.0, 1e6, math.inf, -61440.0, -math.inf])
    assert oracle.e5m2_encode(big).tolist() == [0x7B, 0x7B, 0x7B, 0x7B, 0x7B, 0xFB, 0xFB]
    assert (int(oracle.e5m2_encode([math.nan])[0]) & 0x7C) == 0x7C
    assert int(oracle.e5m2_encode([math.nan])[0]) & 0x03


def test_e5m2_roundtrip_all_finite_codes():
    codes = np.array(FINITE_E5M2, dtype=np.uint8)
    assert np.array_equal(oracle.e5m2_encode(oracle.e5m2_value(codes)), codes)


def _e8m0_brute(amax: float, top: int) -> int:
    if amax == 0:
        return -127
    a = Fraction(amax)
    for e in range(-220, 200):
        if Fraction(top) * (Fraction(2) ** e) >= a:
            return max(-127, min(127, e))
    raise AssertionError("unreachable")


def test_e8m0_e5m2_boundaries_brute_force():
    vals = [0.0, 1.0, 1.75, 2.0, 28672.0, 57343.99, 57344.0, 57344.01]
    for k in range(-160, 113):
        x = math.ldexp(E5M2_MAX, k)
        for v in (x, np.nextafter(x, 0.0), np.nextafter(x, np.inf)):
            v32 = float(np.float32(v))
            if 0.0 < v32 < 3.4e38:
                vals.append(v32)
    got = oracle.e8m0_exponent_e5m2(np.array(vals))
    assert np.array_equal(got, np.array([_e8m0_brute(v, 57344) for v in vals]))


def _torch_quantize(x32, top, dtype):
    """Independent quantiser for a format with largest finite `top`."""
    x = torch.from_numpy(x32.astype(np.float32))
    rows, cols = x.shape
    blk = x.reshape(rows, cols // 32, 32).to(torch.float64)
    amax = blk.abs().amax(dim=-1)
    e = torch.ceil(torch.log2(amax / top))
    e = torch.nan_to_num(torch.where(amax > 0, e, torch.full_like(e, -127.0)), nan=-127.0, neginf=-127.0)
    two = torch.tensor(2.0, dtype=torch.float64)
    e = e + ((top * torch.pow(two, e)) < amax).to(e.dtype)
    e = e - (((top * torch.pow(two, e - 1)) >= amax) & (amax > 0)).to(e.dtype)
    e = e.clamp(-127, 127)
    y = (blk * torch.pow(two, -e).unsqueeze(-1)).clamp(-top, top).to(torch.float32)
    q = y.reshape(rows, cols).to(dtype).view(torch.uint8).numpy()
    return q, (e + 127).to(torch.uint8).numpy()


@pytest.mark.parametrize("name", ["tiny_m128_n256_k512", "skinny_m64_n2048_k7168"])
def test_quantizer_e5m2_matches_torch_path(name):
    w = inputs.WORKLOADS[name]
    a32, b32 = inputs.fp32_operands(w)
    x = np.concatenate([a32, b32[:, : a32.shape[1]]], axis=0)
    x[0, :32] = 0.0
    x[1, 32:64] = E5M2_MAX
    x[2, 64:96] *= 1e4
    q, s = oracle.quantize_mxfp8(x, fmt="e5m2")
    qr, sr = _torch_quantize(x, E5M2_MAX, torch.float8_e5m2)
    assert np.array_equal(s, sr)
    assert np.array_equal(q, qr)
    assert s[1, 1] == 127


def _deq(code, sbyte, fmt):
    return Fraction(float(_torch_value([code], fmt)[0])) * (Fraction(2) ** (sbyte - 127))


@pytest.mark.parametrize("fa,fb", [(oracle.E4M3, oracle.E5M2), (oracle.E5M2, oracle.E4M3),
                                   (oracle.E5M2, oracle.E5M2)])
@pytest.mark.parametrize("R,M,N,kpr,seed", [(1, 2, 2, 32, 21), (2, 2, 3, 32, 22), (3, 2, 2, 64, 23)])
def test_mixed_format_gemm_exact_rational(fa, fb, R, M, N, kpr, seed):
    K = R * kpr
    a = inputs.random_codes((R, M, kpr), seed, FINITE_E5M2 if fa else FINITE_E4M3)
    sa = inputs.random_scale_bytes((R, M, kpr // 32), seed + 1, 118, 132)
    b = inputs.random_codes((N, K), seed + 2, FINITE_E5M2 if fb else FINITE_E4M3)
    sb = inputs.random_scale_bytes((N, K // 32), seed + 3, 118, 132)
    got = oracle.mxgemm_seg(a, sa, b, sb, fmt_a=fa, fmt_b=fb)
    for m in range(M):
        for n in range(N):
            acc, mag = Fraction(0), Fraction(0)
            for r in range(R):
                for k in range(kpr):
                    kg = r * kpr + k
                    t = _deq(int(a[r, m, k]), int(sa[r, m, k // 32]), fa) * \
                        _deq(int(b[n, kg]), int(sb[n, kg // 32]), fb)
                    acc += t
                    mag += abs(t)
            exp = _bf16_rne_fraction(acc)
            if int(got[m, n]) != exp:
                assert _near_midpoint(acc, Fraction(K) * Fraction(1, 2 ** 53) * mag)


def test_mixed_format_gemm_matches_numpy_float64():
    R, M, N, kpr = 2, 24, 40, 64
    K = R * kpr
    a = inputs.random_codes((R, M, kpr), 31, FINITE_E5M2)
    sa = inputs.random_scale_bytes((R, M, kpr // 32), 32, 125, 129)
    b = inputs.random_codes((N, K), 33, FINITE_E4M3)
    sb = inputs.random_scale_bytes((N, K // 32), 34, 125, 129)
    got = oracle.bf16_bits_to_float(oracle.mxgemm_seg(a, sa, b, sb, fmt_a="e5m2", fmt_b="e4m3"))
    av = _torch_value(a, oracle.E5M2) * np.exp2(np.repeat(sa.astype(np.float64) - 127, 32, axis=2))
    A = np.concatenate([av[r] for r in range(R)], axis=1)          # [M, K]
    B = _torch_value(b, oracle.E4M3) * np.exp2(np.repeat(sb.astype(np.float64) - 127, 32, axis=1))
    ref = torch.from_numpy(A @ B.T).to(torch.bfloat16).to(torch.float32).numpy()
    # double rounding through numpy's sum order can differ in the last bf16 bit
    close = np.abs(got - ref) <= np.abs(ref) * 2.0 ** -7
    assert close.all()
    # reading B as the wrong format changes the result: the format is used
    wrong = oracle.bf16_bits_to_float(oracle.mxgemm_seg(a, sa, b, sb, fmt_a="e5m2", fmt_b="e5m2"))
    assert not np.allclose(wrong, got)
