"""CPU oracle for the segmented MXFP8 GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never does; the two
share no code.  The arithmetic lives in ``mxfp8_oracle.c`` (plain C, double
precision, one plainly ordered loop per output); this module only marshals
numpy arrays to it.  See the header of ``mxfp8_oracle.c`` for the definition
and the passages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxfp8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, no floating-point contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                        "-fno-fast-math", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        lib.oracle_e8m0_exponent.restype = ctypes.c_int
        lib.oracle_e8m0_exponent.argtypes = [ctypes.c_double]
        lib.oracle_bf16_from_double.restype = ctypes.c_uint16
        lib.oracle_bf16_from_double.argtypes = [ctypes.c_double]
        lib.oracle_quantize_mx.argtypes = [_f32p, _i64, _i64, _u8p, _u8p, ctypes.c_int]
        lib.oracle_mxgemm_seg.argtypes = [_u8p, _u8p, _u8p, _u8p, _i64, _i64, _i64, _i64, _u16p,
                                          ctypes.c_int, ctypes.c_int]
        lib.oracle_mxgemm_seg_entries.argtypes = [_u8p, _u8p, _u8p, _u8p, _i64, _i64, _i64, _i64,
                                                  _i64p, _i64p, _i64, _u16p, _f64p,
                                                  ctypes.c_int, ctypes.c_int]
        lib.oracle_mxgemm_seg_rows.argtypes = [_u8p, _u8p, _u8p, _u8p, _i64, _i64, _i64, _i64,
                                               _i64, _i64, _u16p, ctypes.c_int, ctypes.c_int]
        lib.oracle_e5m2_encode_array.argtypes = [_f64p, _i64, _u8p]
        lib.oracle_e5m2_value_array.argtypes = [_u8p, _i64, _f64p]
        lib.oracle_e8m0_exponent_e5m2_array.argtypes = [_f64p, _i64, _i32p]
        lib.oracle_e4m3_encode_array.argtypes = [_f64p, _i64, _u8p]
        lib.oracle_e4m3_value_array.argtypes = [_u8p, _i64, _f64p]
        lib.oracle_e8m0_exponent_array.argtypes = [_f64p, _i64, _i32p]
        lib.oracle_bf16_from_double_array.argtypes = [_f64p, _i64, _u16p]
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def e4m3_value(codes) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8).ravel())
    out = np.empty(c.size, dtype=np.float64)
    _load().oracle_e4m3_value_array(_p(c, _u8p), c.size, _p(out, _f64p))
    return out.reshape(np.shape(codes))


def e4m3_encode(values) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float64).ravel())
    out = np.empty(v.size, dtype=np.uint8)
    _load().oracle_e4m3_encode_array(_p(v, _f64p), v.size, _p(out, _u8p))
    return out.reshape(np.shape(values))


def e8m0_exponent(amax) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(amax, dtype=np.float64).ravel())
    out = np.empty(v.size, dtype=np.int32)
    _load().oracle_e8m0_exponent_array(_p(v, _f64p), v.size, _p(out, _i32p))
    return out.reshape(np.shape(amax))


# format codes of the FP8 operands
E4M3, E5M2 = 0, 1


def _fmt(f) -> int:
    if f in (E4M3, "e4m3"):
        return E4M3
    if f in (E5M2, "e5m2"):
        return E5M2
    raise ValueError(f"unknown FP8 format {f!r}")


def e5m2_value(codes) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8).ravel())
    out = np.empty(c.size, dtype=np.float64)
    _load().oracle_e5m2_value_array(_p(c, _u8p), c.size, _p(out, _f64p))
    return out.reshape(np.shape(codes))


def e5m2_encode(values) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float64).ravel())
    out = np.empty(v.size, dtype=np.uint8)
    _load().oracle_e5m2_encode_array(_p(v, _f64p), v.size, _p(out, _u8p))
    return out.reshape(np.shape(values))


def e8m0_exponent_e5m2(amax) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(amax, dtype=np.float64).ravel())
    out = np.empty(v.size, dtype=np.int32)
    _load().oracle_e8m0_exponent_e5m2_array(_p(v, _f64p), v.size, _p(out, _i32p))
    return out.reshape(np.shape(amax))


def bf16_from_double(values) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float64).ravel())
    out = np.empty(v.size, dtype=np.uint16)
    _load().oracle_bf16_from_double_array(_p(v, _f64p), v.size, _p(out, _u16p))
    return out.reshape(np.shape(values))


def quantize_mxfp8(x, fmt=E4M3) -> tuple:
    """``x`` float32 ``[rows, cols]`` (cols % 32 == 0) -> (codes uint8
    ``[rows, cols]`` of format ``fmt``, scale bytes uint8 ``[rows, cols/32]``)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((rows, cols // 32), dtype=np.uint8)
    _load().oracle_quantize_mx(_p(x, _f32p), rows, cols, _p(q, _u8p), _p(s, _u8p), _fmt(fmt))
    return q, s


def _check(a_seg, sa_seg, b, sb):
    a_seg = np.ascontiguousarray(a_seg, dtype=np.uint8)
    sa_seg = np.ascontiguousarray(sa_seg, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    R, M, kpr = a_seg.shape
    N, K = b.shape
    if kpr % 32 or K != R * kpr:
        raise ValueError("inconsistent shapes")
    if sa_seg.shape != (R, M, kpr // 32) or sb.shape != (N, K // 32):
        raise ValueError("inconsistent scale shapes")
    return a_seg, sa_seg, b, sb, R, M, kpr, N


def mxgemm_seg(a_seg, sa_seg, b, sb, fmt_a=E4M3, fmt_b=E4M3) -> np.ndarray:
    """Full C ``[M, N]`` as bfloat16 bit patterns (uint16).

    ``a_seg`` [R, M, kPerRank] codes, ``sa_seg`` [R, M, kPerRank/32] scale
    bytes, ``b`` [N, K] codes, ``sb`` [N, K/32] scale bytes; A codes of
    format ``fmt_a``, B codes of ``fmt_b``."""
    a_seg, sa_seg, b, sb, R, M, kpr, N = _check(a_seg, sa_seg, b, sb)
    c = np.empty((M, N), dtype=np.uint16)
    _load().oracle_mxgemm_seg(_p(a_seg, _u8p), _p(sa_seg, _u8p), _p(b, _u8p), _p(sb, _u8p),
                              R, M, kpr, N, _p(c, _u16p), _fmt(fmt_a), _fmt(fmt_b))
    return c


def mxgemm_seg_entries(a_seg, sa_seg, b, sb, ms, ns, want_exact: bool = False,
                       fmt_a=E4M3, fmt_b=E4M3):
    """C at the listed (ms[i], ns[i]) as bfloat16 bits; optionally also the
    unrounded double sums."""
    a_seg, sa_seg, b, sb, R, M, kpr, N = _check(a_seg, sa_seg, b, sb)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    if ms.shape != ns.shape:
        raise ValueError("ms and ns differ in shape")
    if ms.size and (ms.min() < 0 or ms.max() >= M or ns.min() < 0 or ns.max() >= N):
        raise ValueError("entry index out of range")
    c = np.empty(ms.size, dtype=np.uint16)
    ex = np.empty(ms.size, dtype=np.float64) if want_exact else None
    _load().oracle_mxgemm_seg_entries(_p(a_seg, _u8p), _p(sa_seg, _u8p), _p(b, _u8p),
                                      _p(sb, _u8p), R, M, kpr, N, _p(ms, _i64p), _p(ns, _i64p),
                                      ms.size, _p(c, _u16p),
                                      _p(ex, _f64p) if want_exact else None,
                                      _fmt(fmt_a), _fmt(fmt_b))
    return (c, ex) if want_exact else c


def mxgemm_seg_rows(a_seg, sa_seg, b, sb, m0: int, m1: int, fmt_a=E4M3, fmt_b=E4M3) -> np.ndarray:
    """Rows ``[m0, m1)`` of C as bfloat16 bits."""
    a_seg, sa_seg, b, sb, R, M, kpr, N = _check(a_seg, sa_seg, b, sb)
    if not (0 <= m0 <= m1 <= M):
        raise ValueError("row range out of bounds")
    c = np.empty((m1 - m0, N), dtype=np.uint16)
    _load().oracle_mxgemm_seg_rows(_p(a_seg, _u8p), _p(sa_seg, _u8p), _p(b, _u8p), _p(sb, _u8p),
                                   R, M, kpr, N, m0, m1, _p(c, _u16p), _fmt(fmt_a), _fmt(fmt_b))
    return c


def bf16_bits_to_float(bits) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns (a bit shift)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)
