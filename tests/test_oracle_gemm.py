"""Pins for the oracle's segmented MXFP8 GEMM.

The oracle's product is checked against: exact rational brute force with a
brute-force bfloat16 rounding (tiny shapes), integer closed forms, numpy's
float64 matrix product, the invariance of the result to how K is split into
rank segments, the exact power-of-two scale-shift law, the transpose
identity, and a one-block scale probe.  A dropped term, a wrong segment or
scale index, a transposed operand or a wrong sign fails at least one of
them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_mxgemm_amd import inputs


FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def _deq_fraction(code: int, sbyte: int) -> Fraction:
    v = torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).item()
    return Fraction(v) * (Fraction(2) ** (sbyte - 127))


def _bf16_rne_fraction(x: Fraction) -> int:
    """bfloat16 bits of the exact rational x, round-to-nearest-even, by
    bisection over the enumerated finite bfloat16 grid."""
    neg = x < 0
    a = -x if neg else x
    bits, vals = _bf16_grid_fracs()
    lo, hi = 0, len(vals) - 1
    if a >= vals[-1]:
        top_ulp = vals[-1] - vals[-2]
        r = 0x7F80 if a >= vals[-1] + top_ulp / 2 else int(bits[-1])
        return r | (0x8000 if neg else 0)
    while hi - lo > 1:                       # vals[lo] <= a < vals[hi]
        mid = (lo + hi) // 2
        if vals[mid] <= a:
            lo = mid
        else:
            hi = mid
    dlo, dhi = a - vals[lo], vals[hi] - a
    if dlo < dhi or (dlo == dhi and int(bits[lo]) % 2 == 0):
        r = int(bits[lo])
    else:
        r = int(bits[hi])
    return r | (0x8000 if neg else 0)


_GRID_F = None


def _bf16_grid_fracs():
    global _GRID_F
    if _GRID_F is None:
        b = np.arange(0, 0x7F80, dtype=np.uint32)          # +0 .. largest finite
        v = (b << np.uint32(16)).view(np.float32)
        _GRID_F = (b, [Fraction(float(x)) for x in v])
    return _GRID_F


def _brute_gemm(a_seg, sa_seg, b, sb):
    """Exact rational sum of all terms; returns (bf16 bits of the exact sum,
    bound on how far a double-precision running sum can stray from it)."""
    R, M, kpr = a_seg.shape
    N, K = b.shape
    out = np.empty((M, N), dtype=np.uint16)
    bound = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            mag = Fraction(0)
            for r in range(R):
                for k in range(kpr):
                    kg = r * kpr + k
                    t = (_deq_fraction(int(a_seg[r, m, k]), int(sa_seg[r, m, k // 32]))
                         * _deq_fraction(int(b[n, kg]), int(sb[n, kg // 32])))
                    acc += t
                    mag += abs(t)
            out[m, n] = _bf16_rne_fraction(acc)
            # classic recursive-summation bound: |fl - exact| <= (n-1) u sum|t|
            bound[m, n] = (acc, Fraction(K) * Fraction(1, 2 ** 53) * mag)
    return out, bound


def _near_midpoint(acc: Fraction, tol: Fraction) -> bool:
    """True when a bfloat16 tie lies within tol of acc (then a double sum may
    legitimately round the other way)."""
    for d in (-tol, tol):
        if _bf16_rne_fraction(acc + d) != _bf16_rne_fraction(acc):
            return True
    return False


def _random_case(R, M, N, kpr, seed, slo=120, shi=134):
    K = R * kpr
    a = inputs.random_codes((R, M, kpr), seed, FINITE)
    sa = inputs.random_scale_bytes((R, M, kpr // 32), seed + 1, slo, shi)
    b = inputs.random_codes((N, K), seed + 2, FINITE)
    sb = inputs.random_scale_bytes((N, K // 32), seed + 3, slo, shi)
    return a, sa, b, sb


@pytest.mark.parametrize("R,M,N,kpr,seed", [
    (1, 2, 3, 32, 1), (2, 3, 2, 32, 2), (3, 2, 2, 64, 3), (2, 1, 4, 64, 4), (3, 3, 3, 32, 5),
])
def test_oracle_equals_exact_rational_brute_force(R, M, N, kpr, seed):
    a, sa, b, sb = _random_case(R, M, N, kpr, seed)
    got = oracle.mxgemm_seg(a, sa, b, sb)
    exp, bound = _brute_gemm(a, sa, b, sb)
    undecided = 0
    for (m, n), g in np.ndenumerate(got):
        if g != exp[m, n]:
            acc, tol = bound[m, n]
            assert _near_midpoint(acc, tol), (m, n, hex(g), hex(exp[m, n]))
            undecided += 1
    # for these seeds no sum sits that close to a tie
    assert undecided <= 1


@pytest.mark.parametrize("seed", [41, 42])
def test_oracle_brute_force_narrow_scales_exact(seed):
    # scale bytes in a narrow band: every partial sum is exact in double, so
    # the oracle must equal the correctly rounded exact sum everywhere
    a, sa, b, sb = _random_case(2, 3, 3, 64, seed, slo=126, shi=128)
    a &= np.uint8(0xBF)                     # codes with |value| <= 2^0 * 1.875
    got = oracle.mxgemm_seg(a, sa, b, sb)
    exp, _ = _brute_gemm(a, sa, b, sb)
    assert np.array_equal(got, exp)


def _sign_codes(shape, density, seed):
    """Quantise a {-1,0,+1} matrix with the oracle's quantiser; every
    dequantised value is exactly -1, 0 or +1."""
    x = inputs.sparse_sign_matrix(shape, density, seed)
    q, s = oracle.quantize_mxfp8(x)
    return x, q, s


@pytest.mark.parametrize("R,M,N,kpr,density", [(2, 16, 24, 128, 1.0), (4, 8, 8, 64, 0.5),
                                               (8, 6, 10, 32, 0.9)])
def test_oracle_integer_closed_form(R, M, N, kpr, density):
    K = R * kpr
    xa, qa, sa = _sign_codes((M, K), density, 21 + R)
    xb, qb, sb = _sign_codes((N, K), density, 31 + R)
    a_seg = inputs.split_segments(qa, R)
    sa_seg = inputs.split_segments(sa, R)
    c = oracle.mxgemm_seg(a_seg, sa_seg, qb, sb)
    ref = xa.astype(np.int64) @ xb.astype(np.int64).T          # |ref| <= 256
    assert np.abs(ref).max() <= 256
    ref_bits = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(c, ref_bits)


def test_oracle_all_ones_k256():
    x = np.ones((3, 256), dtype=np.float32)
    q, s = oracle.quantize_mxfp8(x)
    c = oracle.mxgemm_seg(inputs.split_segments(q, 2), inputs.split_segments(s, 2), q, s)
    assert np.all(oracle.bf16_bits_to_float(c) == 256.0)


def test_oracle_k_split_invariance():
    w = inputs.WORKLOADS["skinny_m64_n2048_k7168"]
    a32, b32 = inputs.fp32_operands(w)
    a32, b32 = a32[:8], b32[:16]
    qa, sa = oracle.quantize_mxfp8(a32)
    qb, sb = oracle.quantize_mxfp8(b32)
    outs = []
    for R in (1, 2, 4, 7, 8, 14):
        outs.append(oracle.mxgemm_seg(inputs.split_segments(qa, R), inputs.split_segments(sa, R),
                                      qb, sb))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_oracle_matches_numpy_float64_matmul():
    w = inputs.WORKLOADS["tiny_m128_n256_k512"]
    a32, b32 = inputs.fp32_operands(w)
    qa, sa = oracle.quantize_mxfp8(a32)
    qb, sb = oracle.quantize_mxfp8(b32)
    c = oracle.mxgemm_seg(inputs.split_segments(qa, w.R), inputs.split_segments(sa, w.R), qb, sb)

    def deq(q, s):
        v = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        return v * np.repeat(np.exp2(s.astype(np.float64) - 127.0), 32, axis=1)

    ref = deq(qa, sa) @ deq(qb, sb).T
    got = oracle.bf16_bits_to_float(c).astype(np.float64)
    # the double sums agree to ~1e-15 relative, so the bfloat16 results are
    # the same except where the double value sits within that of a tie
    ulp = np.exp2(np.floor(np.log2(np.abs(ref))) - 7)
    assert np.all(np.abs(got - ref) <= 0.5 * ulp * (1 + 1e-9))
    assert np.mean(c == oracle.bf16_from_double(ref)) > 0.999


def test_oracle_scale_shift_law():
    a, sa, b, sb = _random_case(3, 5, 7, 64, 77)
    c0 = oracle.mxgemm_seg(a, sa, b, sb)
    for t in (-5, 1, 3):
        c1 = oracle.mxgemm_seg(a, (sa.astype(np.int64) + t).astype(np.uint8), b, sb)
        assert np.array_equal(oracle.bf16_bits_to_float(c1),
                              oracle.bf16_bits_to_float(c0) * np.float32(2.0 ** t))


def test_oracle_transpose_identity():
    a, sa, b, sb = _random_case(2, 6, 9, 64, 88)
    R, M, kpr = a.shape
    c = oracle.mxgemm_seg(a, sa, b, sb)
    a_full = np.concatenate(list(a), axis=1)            # [M, K]
    sa_full = np.concatenate(list(sa), axis=1)          # [M, K/32]
    ct = oracle.mxgemm_seg(b[None], sb[None], a_full, sa_full)
    assert np.array_equal(ct.T, c)


def test_oracle_one_block_scale_probe():
    a, sa, b, sb = _random_case(2, 4, 5, 64, 99)
    R, M, kpr = a.shape
    ms, ns = np.meshgrid(np.arange(M), np.arange(b.shape[0]), indexing="ij")
    _, ex0 = oracle.mxgemm_seg_entries(a, sa, b, sb, ms.ravel(), ns.ravel(), want_exact=True)
    r, m, blk, t = 1, 2, 1, 4
    sa2 = sa.copy()
    sa2[r, m, blk] += t
    _, ex1 = oracle.mxgemm_seg_entries(a, sa2, b, sb, ms.ravel(), ns.ravel(), want_exact=True)
    d = (ex1 - ex0).reshape(M, -1)
    assert np.all(d[np.arange(M) != m] == 0)
    # the change in row m is (2^t - 1) times that block's contribution
    av = torch.from_numpy(a[r, m, blk * 32:(blk + 1) * 32].copy()).view(torch.float8_e4m3fn).double().numpy()
    av = av * 2.0 ** (int(sa[r, m, blk]) - 127)
    kg = r * kpr + blk * 32
    bv = torch.from_numpy(b[:, kg:kg + 32].copy()).view(torch.float8_e4m3fn).double().numpy()
    bv = bv * np.exp2(sb[:, kg // 32].astype(np.float64) - 127.0)[:, None]
    contrib = bv @ av
    assert np.allclose(d[m], (2.0 ** t - 1) * contrib, rtol=1e-12, atol=0)


def test_oracle_entries_and_rows_agree_with_full():
    a, sa, b, sb = _random_case(3, 9, 11, 96, 123)
    c = oracle.mxgemm_seg(a, sa, b, sb)
    rng = np.random.default_rng(0)
    ms = rng.integers(0, 9, 40)
    ns = rng.integers(0, 11, 40)
    assert np.array_equal(oracle.mxgemm_seg_entries(a, sa, b, sb, ms, ns), c[ms, ns])
    assert np.array_equal(oracle.mxgemm_seg_rows(a, sa, b, sb, 2, 7), c[2:7])


def test_oracle_rejects_bad_shapes():
    a, sa, b, sb = _random_case(2, 3, 4, 64, 1)
    with pytest.raises(ValueError):
        oracle.mxgemm_seg(a, sa, b[:, :64], sb)
    with pytest.raises(ValueError):
        oracle.mxgemm_seg_entries(a, sa, b, sb, [5], [0])
