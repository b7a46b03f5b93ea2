"""Seeded random problem shapes for the plan and parity sweeps (imported by
test modules, not collected): rank count, rows, K per rank (a multiple of
the 128-wide K-step), N, chunk rows (commMSize need not divide M) and ring
depth (a power of two)."""
import numpy as np


def random_shapes(seed, count, max_m=400, max_n=300, max_k=4096):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        R = int(rng.integers(1, 9))
        kpr = 128 * int(rng.integers(1, 5))
        if R * kpr > max_k:
            continue
        M = int(rng.integers(1, max_m + 1))
        cms = int(rng.integers(1, M + 1)) if rng.random() < 0.7 else int(rng.integers(1, 65))
        nbuf = int(2 ** rng.integers(0, 4))
        N = int(rng.integers(1, max_n + 1))
        out.append((R, M, kpr, N, cms, nbuf))
    return out
