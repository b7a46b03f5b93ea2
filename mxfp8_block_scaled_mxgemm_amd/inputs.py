"""Seeded synthetic inputs for the segmented MXFP8 GEMM.

This module only draws random numbers and lays them out.  It holds none of
the method's arithmetic: no FP8 or E8M0 encoding, no scaling, no products.
Both the CPU oracle (in tests) and the HIP path (tests, bench) take their
inputs from here, so neither side depends on the other.

Problem statement followed (cannbot-harness 0.1.5 package diff,
all_to_all_matmul.cpp, argument parsing and host buffer sizing): every one of
``R`` ranks holds A as ``R`` segments of ``[M, kPerRank]``; the full K is
``R * kPerRank``; B is held transposed as ``[N, K]`` (the kernel entry sets
TransB, all_to_all_matmul_impl.h, kernel entries).

The five workloads below are the sizes this library is measured on; a
sixth is the source's own example shape.  Each is
drawn from ``numpy.random.default_rng(seed)`` (PCG64) as fp32 normals; the
outlier workload then multiplies an independent 1 % of A's entries, and then
of B's, by 100.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    R: int            # simulated ranks = K segments
    M: int            # rows of A and C
    kPerRank: int     # K columns per segment
    N: int            # columns of C (rows of the [N, K] B)
    commMSize: int    # rows per staged chunk
    nbuf: int         # staging ring depth
    sigma: float      # standard deviation of the normals
    outlier_frac: float
    outlier_mul: float
    seed: int

    @property
    def K(self) -> int:
        return self.R * self.kPerRank

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """A + A scales + B + B scales + C, each counted once (1 B per FP8
        code, 1 B per E8M0 scale, 2 B per BF16 output)."""
        K = self.K
        return (self.M * K + self.M * K // 32 + self.N * K + self.N * K // 32
                + 2 * self.M * self.N)

    def describe(self) -> str:
        return (f"R={self.R} M={self.M} kPerRank={self.kPerRank} K={self.K} "
                f"N={self.N} commMSize={self.commMSize} nbuf={self.nbuf}")


WORKLOADS: Dict[str, Workload] = {
    "tiny_m128_n256_k512": Workload("tiny_m128_n256_k512", 2, 128, 256, 256, 64, 2, 1.0, 0.0, 1.0, 101),
    "m1024_n2048_k4096": Workload("m1024_n2048_k4096", 4, 1024, 1024, 2048, 256, 2, 1.0, 0.0, 1.0, 102),
    "m4096_n4096_k7168": Workload("m4096_n4096_k7168", 8, 4096, 896, 4096, 512, 4, 0.5, 0.0, 1.0, 103),
    "skinny_m64_n2048_k7168": Workload("skinny_m64_n2048_k7168", 8, 64, 896, 2048, 8, 4, 1.0, 0.0, 1.0, 104),
    "outlier_m8192_n8192_k8192": Workload("outlier_m8192_n8192_k8192", 8, 8192, 1024, 8192, 512, 4, 1.0, 0.01, 100.0, 105),
    # the performance example of the source's host program (m 2048, k 8192,
    # n 3584, 4 ranks) with its chunk size 512 and ring depth 4
    "example_m2048_n3584_k8192": Workload("example_m2048_n3584_k8192", 4, 2048, 2048, 3584, 512, 4, 1.0, 0.0, 1.0, 106),
}


def fp32_operands(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Return ``(A32 [M, K], Bt32 [N, K])`` as C-contiguous float32.

    B is drawn directly in its stored ``[N, K]`` orientation; its entries are
    iid, so this is the same distribution as drawing ``[K, N]``.
    """
    rng = np.random.default_rng(w.seed)
    a = rng.standard_normal((w.M, w.K), dtype=np.float32)
    b = rng.standard_normal((w.N, w.K), dtype=np.float32)
    if w.sigma != 1.0:
        a *= np.float32(w.sigma)
        b *= np.float32(w.sigma)
    if w.outlier_frac > 0.0:
        mask = rng.random((w.M, w.K)) < w.outlier_frac
        a[mask] *= np.float32(w.outlier_mul)
        del mask
        mask = rng.random((w.N, w.K)) < w.outlier_frac
        b[mask] *= np.float32(w.outlier_mul)
        del mask
    return np.ascontiguousarray(a), np.ascontiguousarray(b)


def random_codes(shape, seed: int, choices=None) -> np.ndarray:
    """Uniform random bytes (uint8).  ``choices`` restricts them to a given
    list of byte values (for example codes whose values are small integers,
    or finite codes only)."""
    rng = np.random.default_rng(seed)
    if choices is None:
        return rng.integers(0, 256, size=shape, dtype=np.uint8)
    choices = np.asarray(choices, dtype=np.uint8)
    return choices[rng.integers(0, len(choices), size=shape)]


def random_scale_bytes(shape, seed: int, lo: int, hi: int) -> np.ndarray:
    """Uniform random bytes in ``[lo, hi]`` (uint8)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape, dtype=np.uint8)


def sparse_sign_matrix(shape, density: float, seed: int) -> np.ndarray:
    """float32 matrix with entries in {-1, 0, +1}: each entry is non-zero with
    probability ``density`` and then +1 or -1 with equal odds."""
    rng = np.random.default_rng(seed)
    nz = rng.random(shape) < density
    sign = np.where(rng.random(shape) < 0.5, np.float32(-1.0), np.float32(1.0))
    return np.where(nz, sign, np.float32(0.0)).astype(np.float32)


def split_segments(full: np.ndarray, R: int) -> np.ndarray:
    """Re-lay a ``[M, R*w]`` row-major array as ``[R, M, w]``: segment r is
    columns ``[r*w, (r+1)*w)``.  This is the sender-side layout of A (segment
    r is meant for rank r; all_to_all_comm_udma.h, PutSegmentToRank source
    offset)."""
    M, cols = full.shape
    assert cols % R == 0
    w = cols // R
    return np.ascontiguousarray(full.reshape(M, R, w).transpose(1, 0, 2))
