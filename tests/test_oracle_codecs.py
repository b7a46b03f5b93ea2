"""Pins for the oracle's encodings: E4M3FN decode/encode, the E8M0 exponent
rule, the MXFP8 block quantiser and the double -> bfloat16 rounding.

Each check compares the oracle with something other than itself: a library
routine (torch's float8_e4m3fn and bfloat16 casts), the OCP spec points in
tests/golden/, brute-force searches written from the definitions, or
invariants of the encoding.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_mxgemm_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_points(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                a, b = line.split()
                rows.append((int(a, 16), b))
    return rows


def _torch_e4m3_value(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_e4m3_encode(f32):
    t = torch.from_numpy(np.asarray(f32, dtype=np.float32).copy())
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ----------------------------------------------------------------- decode --

def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_value(codes)
    ref = _torch_e4m3_value(codes)
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert np.array_equal(nan_ours, nan_ref)
    assert set(np.nonzero(nan_ours)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan_ours], ref[~nan_ref])
    # signed zero kept
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3_decode_spec_points():
    for code, val in _read_points("e4m3fn_spec_points.txt"):
        got = float(oracle.e4m3_value([code])[0])
        if val == "nan":
            assert math.isnan(got), hex(code)
        else:
            assert got == float(val), hex(code)
            assert math.copysign(1.0, got) == math.copysign(1.0, float(val))


# ----------------------------------------------------------------- encode --

def _structured_fp32():
    """fp32 values with |v| <= 448: every (sign, exponent, top 7 mantissa
    bits) combination, each with low-16-bit patterns that include exact
    ties and their neighbours."""
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000,
                     0x2345], dtype=np.uint32)
    exps = np.arange(0, 136, dtype=np.uint32)      # biased; 135 -> [256, 512)
    top = np.arange(128, dtype=np.uint32)
    sign = np.array([0, 1], dtype=np.uint32)
    g = np.meshgrid(sign, exps, top, lows, indexing="ij")
    bits = (g[0] << 31) | (g[1] << 23) | (g[2] << 16) | g[3]
    f = bits.ravel().view(np.float32)
    return f[np.abs(f) <= np.float32(448.0)]


def test_e4m3_encode_matches_torch_structured():
    f = _structured_fp32()
    ours = oracle.e4m3_encode(f.astype(np.float64))
    ref = _torch_e4m3_encode(f)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(float(f[i]), hex(ours[i]), hex(ref[i])) for i in bad[:10]]


def test_e4m3_encode_matches_torch_random():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) <= np.float32(448.0))]
    ours = oracle.e4m3_encode(f.astype(np.float64))
    ref = _torch_e4m3_encode(f)
    assert np.array_equal(ours, ref)


def _exhaustive_encode_check(encode, torch_dtype, limit_bits, chunk=1 << 26):
    """Every fp32 bit pattern with |v| <= the format's largest finite value
    (both signs), in chunks: the oracle's encoder against torch's cast."""
    for sign in (0, 0x80000000):
        for lo in range(0, limit_bits + 1, chunk):
            hi = min(lo + chunk, limit_bits + 1)
            bits = np.arange(lo, hi, dtype=np.uint32) | np.uint32(sign)
            f = bits.view(np.float32)
            ref = torch.from_numpy(f).to(torch_dtype).view(torch.uint8).numpy()
            ours = encode(f.astype(np.float64))
            if not np.array_equal(ours, ref):
                i = int(np.nonzero(ours != ref)[0][0])
                raise AssertionError(f"{float(f[i])!r} (bits {int(bits[i]):#010x}): oracle {int(ours[i]):#04x}, "
                                     f"torch {int(ref[i]):#04x}")


def test_e4m3_encode_exhaustive_matches_torch():
    """All 2 x 1.14e9 fp32 values with |v| <= 448 (0x43E00000)."""
    _exhaustive_encode_check(oracle.e4m3_encode, torch.float8_e4m3fn, 0x43E00000)


def test_e4m3_encode_decode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_value(codes)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


# ------------------------------------------------------------------- E8M0 --

def _e8m0_brute(amax: float) -> int:
    """Smallest integer e with 448 * 2^e >= amax, by exhaustive search with
    exact rationals, then clamped to [-127, 127] (0 -> -127)."""
    if amax == 0:
        return -127
    a = Fraction(amax)
    for e in range(-200, 200):
        if Fraction(448) * (Fraction(2) ** e) >= a:
            return max(-127, min(127, e))
    raise AssertionError("unreachable")


def test_e8m0_exponent_boundaries_brute_force():
    vals = [0.0]
    for k in range(-150, 129):
        x = math.ldexp(448.0, k)
        for v in (x, np.nextafter(x, 0.0), np.nextafter(x, np.inf)):
            if v < 3.4e38:
                v32 = float(np.float32(v))
                if 0.0 < v32 < 3.4e38:
                    vals.append(v32)
    vals += [float(np.float32(v)) for v in (1.0, 2.0, 3.5, 223.99, 224.0, 224.01, 447.99)]
    vals += [float(np.float32(x)) for x in (1e-45, 1e-40, 1.17549435e-38)]
    got = oracle.e8m0_exponent(np.array(vals))
    exp = np.array([_e8m0_brute(v) for v in vals])
    assert np.array_equal(got, exp)


def test_e8m0_spec_points():
    # the scale byte is e + 127 (OCP MX, E8M0 bias 127)
    for byte, log2v in _read_points("e8m0_spec_points.txt"):
        e = int(log2v)
        assert byte == e + 127
        # an amax of exactly 448 * 2^e must map to that byte
        if -127 <= e <= 126:
            assert oracle.e8m0_exponent([math.ldexp(448.0, e)])[0] + 127 == byte


def test_e8m0_matches_float_log2_off_boundary():
    rng = np.random.default_rng(3)
    amax = np.exp(rng.uniform(-60, 60, size=200000)).astype(np.float32).astype(np.float64)
    t = np.log2(amax / 448.0)
    safe = np.abs(t - np.round(t)) > 1e-9
    ref = np.clip(np.ceil(t[safe]), -127, 127).astype(np.int32)
    got = oracle.e8m0_exponent(amax[safe])
    assert np.array_equal(got, ref)


# -------------------------------------------------------------- quantiser --

def _torch_quantize(x32: np.ndarray):
    """Independent quantiser: exponent from float64 log2 corrected by exact
    power-of-two comparisons, codes from torch's float8_e4m3fn cast."""
    x = torch.from_numpy(x32.astype(np.float32))
    rows, cols = x.shape
    blk = x.reshape(rows, cols // 32, 32).to(torch.float64)
    amax = blk.abs().amax(dim=-1)
    e = torch.ceil(torch.log2(amax / 448.0))
    e = torch.where(amax > 0, e, torch.full_like(e, -127.0))
    e = torch.nan_to_num(e, nan=-127.0, neginf=-127.0)
    # fix the float log2 at exact boundaries: enforce the defining property
    two = torch.tensor(2.0, dtype=torch.float64)
    too_small = (448.0 * torch.pow(two, e)) < amax
    e = e + too_small.to(e.dtype)
    too_big = (448.0 * torch.pow(two, e - 1)) >= amax
    e = e - (too_big & (amax > 0)).to(e.dtype)
    e = e.clamp(-127, 127)
    y = (blk * torch.pow(two, -e).unsqueeze(-1)).to(torch.float32)
    q = y.reshape(rows, cols).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    s = (e + 127).to(torch.uint8).numpy()
    return q, s


@pytest.mark.parametrize("name", ["tiny_m128_n256_k512", "skinny_m64_n2048_k7168"])
def test_quantizer_matches_torch_path(name):
    w = inputs.WORKLOADS[name]
    a32, b32 = inputs.fp32_operands(w)
    for x in (a32, b32):
        q, s = oracle.quantize_mxfp8(x)
        qr, sr = _torch_quantize(x)
        assert np.array_equal(s, sr)
        assert np.array_equal(q, qr)


def test_quantizer_outliers_and_edges_match_torch_path():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    x[rng.random(x.shape) < 0.02] *= 100.0
    x[3, :32] = 0.0                         # all-zero block
    x[4, 32:64] = -0.0                      # negative zeros
    x[5, 64:96] = 448.0                     # amax exactly 448 -> e = 0
    x[6, 96:128] = np.float32(448.0) * np.float32(2.0 ** -20)
    x[7, 128:160] = np.float32(1e-39)       # subnormal fp32 amax
    x[8, 160:192] = np.float32(3.0e38)      # huge amax
    x[9, 192:224] = np.linspace(-1, 1, 32, dtype=np.float32) * np.float32(2.0 ** -130)
    q, s = oracle.quantize_mxfp8(x)
    qr, sr = _torch_quantize(x)
    assert np.array_equal(s, sr)
    assert np.array_equal(q, qr)
    assert s[5, 2] == 127 and s[3, 0] == 0
    assert np.all(q[4, 32:64] == 0x80)      # sign of zero kept


def test_quantizer_invariants():
    w = inputs.WORKLOADS["tiny_m128_n256_k512"]
    a32, _ = inputs.fp32_operands(w)
    q, s = oracle.quantize_mxfp8(a32)
    assert not np.any((q & 0x7F) == 0x7F)              # never NaN
    e = s.astype(np.int64) - 127
    blk = a32.reshape(a32.shape[0], -1, 32).astype(np.float64)
    amax = np.abs(blk).max(axis=-1)
    ratio = amax * np.exp2(-e)
    assert np.all((ratio > 224.0) & (ratio <= 448.0))   # scale is tight
    deq = oracle.e4m3_value(q).reshape(blk.shape) * np.exp2(e)[..., None]
    err = np.abs(deq - blk)
    y = np.abs(blk) * np.exp2(-e)[..., None]
    # half a step of the E4M3 grid at |y|, times the block scale
    step = np.where(y < 2.0 ** -6, 2.0 ** -9,
                    np.exp2(np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3))
    assert np.all(err <= 0.5 * step * np.exp2(e)[..., None] * (1 + 1e-12))
    assert np.all(np.sign(deq) * np.sign(blk) >= 0)


# ------------------------------------------------------------------- BF16 --

def _bf16_grid():
    bits = np.arange(0, 0x7F81, dtype=np.uint32)          # +0 .. +inf
    vals = (bits << np.uint32(16)).view(np.float32).astype(np.float64)
    return bits.astype(np.uint16), vals


_GRID = None


def _bf16_brute(v: float) -> int:
    """Round-to-nearest-even onto the bfloat16 grid by bisection over the
    enumerated non-negative bfloat16 values (exact rational comparisons)."""
    global _GRID
    if _GRID is None:
        _GRID = _bf16_grid()
    bits, vals = _GRID
    neg = math.copysign(1.0, v) < 0
    a = abs(v)
    i = int(np.searchsorted(vals, a, side="left"))
    if i < len(vals) and vals[i] == a:
        r = int(bits[i])
    else:
        lo, hi = i - 1, i
        dlo = Fraction(a) - Fraction(float(vals[lo]))
        if hi >= len(vals) - 1:                 # beyond the largest finite
            top = Fraction(float(vals[-2]))
            ulp = top - Fraction(float(vals[-3]))
            r = int(bits[-1]) if Fraction(a) >= top + ulp / 2 else int(bits[-2])
        else:
            dhi = Fraction(float(vals[hi])) - Fraction(a)
            if dlo < dhi:
                r = int(bits[lo])
            elif dhi < dlo:
                r = int(bits[hi])
            else:
                r = int(bits[lo]) if int(bits[lo]) % 2 == 0 else int(bits[hi])
    return r | (0x8000 if neg else 0)


def test_bf16_from_float_representable_matches_torch():
    rng = np.random.default_rng(5)
    b = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    b[: 1 << 16] = (b[: 1 << 16] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)   # exact ties
    f = b.view(np.float32)
    f = f[np.isfinite(f)]
    ours = oracle.bf16_from_double(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_from_double_brute_force():
    rng = np.random.default_rng(9)
    vals = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 130, 3000)))
    # double-rounding traps: just above / below a bfloat16 midpoint, off the
    # float32 grid
    for k in (-130, -127, -20, 0, 7, 100, 127):
        mid = math.ldexp(1.0 + 2.0 ** -8, k)
        vals += [mid, mid + math.ldexp(1.0, k - 40), mid - math.ldexp(1.0, k - 40)]
    vals += [3.3895313892515355e38, 3.3961e38, 3.4e38, 5e-324, 1e-45, 0.0, -0.0]
    got = oracle.bf16_from_double(np.array(vals))
    exp = np.array([_bf16_brute(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, exp), [(v, hex(g), hex(e)) for v, g, e in zip(vals, got, exp) if g != e][:5]
    # the classic trap: 1 + 2^-8 + 2^-40 must round up, not to 1.0
    assert oracle.bf16_from_double([1.0 + 2.0 ** -8 + 2.0 ** -40])[0] == 0x3F81
