"""ctypes binding of ``libmxgemm_seg.so`` (declared in ``include/mxgemm_seg.h``).

Argument marshalling only: every step of the GEMM path runs in the HIP
library.  torch supplies device memory and streams.  If the library is
missing this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmxgemm_seg.so")

MXGEMM_OK = 0
MXGEMM_EINVAL = -1
MXGEMM_ENOMEM = -2
MXGEMM_EHIP = -3
MXGEMM_EUNSUPPORTED = -4
MXGEMM_ETIMEOUT = -5
_NAMES = {MXGEMM_EINVAL: "EINVAL", MXGEMM_ENOMEM: "ENOMEM", MXGEMM_EHIP: "EHIP",
          MXGEMM_EUNSUPPORTED: "EUNSUPPORTED", MXGEMM_ETIMEOUT: "ETIMEOUT"}

EXPORTED = [
    "mxgemm_seg_create", "mxgemm_seg_create_ex", "mxgemm_seg_run", "mxgemm_seg_destroy",
    "mxgemm_seg_last_error", "mxgemm_seg_get_plan", "mxgemm_seg_plan", "mxgemm_seg_decode",
    "mxgemm_quantize_mxfp8", "mxgemm_quantize_mx", "mxgemm_seg_set_profiling",
    "mxgemm_seg_kernel_times", "mxgemm_seg_status", "mxgemm_seg_run_static",
]


class MxgemmError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


class Plan(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("kPerRank", ctypes.c_int64), ("N", ctypes.c_int64),
        ("K", ctypes.c_int64), ("commMSize", ctypes.c_int64),
        ("rank_size", ctypes.c_int32), ("buffer_count", ctypes.c_int32),
        ("chunks", ctypes.c_int32), ("chunks_per_window", ctypes.c_int32),
        ("windows", ctypes.c_int32), ("window_slots", ctypes.c_int32),
        ("tile_cfg", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
        ("split", ctypes.c_int32), ("tiles_m", ctypes.c_int32), ("tiles_n", ctypes.c_int32),
        ("work_items", ctypes.c_int32), ("grid", ctypes.c_int32), ("group_n", ctypes.c_int32),
        ("num_cus", ctypes.c_int32), ("precision", ctypes.c_int32),
        ("a_format", ctypes.c_int32), ("b_format", ctypes.c_int32),
        ("ring", ctypes.c_int32), ("spin_limit", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("slot_bytes", ctypes.c_int64), ("scale_slot_bytes", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


PRECISION_EXACT = 0
PRECISION_NATIVE = 1
FMT_E4M3 = 0
FMT_E5M2 = 1
RING_EVENTS = 0
RING_FLAGS = 1


def _fmt(f) -> int:
    """Format code of ``f`` (a code, "e4m3"/"e5m2", or -1/None for the default)."""
    if f is None or f == -1:
        return -1
    if isinstance(f, str):
        return {"e4m3": FMT_E4M3, "e5m2": FMT_E5M2}[f.lower()]
    return int(f)


class Options(ctypes.Structure):
    _fields_ = [("tile_cfg", ctypes.c_int32), ("split", ctypes.c_int32),
                ("chunks_per_window", ctypes.c_int32),
                ("precision", ctypes.c_int32),
                ("a_format", ctypes.c_int32), ("b_format", ctypes.c_int32),
                ("ring", ctypes.c_int32), ("spin_limit", ctypes.c_int32)]


def _ring(r) -> int:
    if r is None or r == -1:
        return -1
    if isinstance(r, str):
        return {"events": RING_EVENTS, "flags": RING_FLAGS}[r.lower()]
    return int(r)


def options(tile_cfg=-1, split=-1, chunks_per_window=-1, precision=-1, a_format=-1,
            b_format=-1, ring=-1, spin_limit=-1) -> Options:
    return Options(tile_cfg, split, chunks_per_window, precision, _fmt(a_format), _fmt(b_format),
                   _ring(ring), spin_limit)


_lib = None


def load():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mxfp8_block_scaled_mxgemm_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.mxgemm_seg_create.argtypes = [ctypes.POINTER(vp), i64, i64, i32, i64, i64, i32]
    lib.mxgemm_seg_create_ex.argtypes = [ctypes.POINTER(vp), i64, i64, i32, i64, i64, i32,
                                         ctypes.POINTER(Options)]
    lib.mxgemm_seg_run.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.mxgemm_seg_run_static.argtypes = [i64, i64, i32, i64, i64, i32, ctypes.POINTER(Options),
                                          vp, vp, vp, vp, vp, vp]
    lib.mxgemm_seg_destroy.argtypes = [vp]
    lib.mxgemm_seg_last_error.restype = ctypes.c_char_p
    lib.mxgemm_seg_get_plan.argtypes = [vp, ctypes.POINTER(Plan)]
    lib.mxgemm_seg_plan.argtypes = [ctypes.POINTER(Plan), i64, i64, i32, i64, i64, i32, i32,
                                    ctypes.POINTER(Options)]
    p32 = ctypes.POINTER(i32)
    lib.mxgemm_seg_decode.argtypes = [ctypes.POINTER(Plan), i64, i32, i32, p32, p32, p32, p32]
    lib.mxgemm_quantize_mxfp8.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, vp]
    lib.mxgemm_quantize_mx.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, i32, vp]
    lib.mxgemm_seg_set_profiling.argtypes = [vp, i32]
    lib.mxgemm_seg_status.argtypes = [vp]
    lib.mxgemm_seg_kernel_times.argtypes = [vp, ctypes.POINTER(ctypes.c_double), p32,
                                            ctypes.POINTER(ctypes.c_double), p32]
    for name in ("mxgemm_seg_create", "mxgemm_seg_create_ex", "mxgemm_seg_run",
                 "mxgemm_seg_destroy", "mxgemm_seg_get_plan", "mxgemm_seg_plan",
                 "mxgemm_seg_decode", "mxgemm_quantize_mxfp8", "mxgemm_quantize_mx",
                 "mxgemm_seg_set_profiling", "mxgemm_seg_status",
                 "mxgemm_seg_kernel_times", "mxgemm_seg_run_static"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def check(rc: int):
    if rc != MXGEMM_OK:
        raise MxgemmError(rc, load().mxgemm_seg_last_error().decode())


def last_error() -> str:
    return load().mxgemm_seg_last_error().decode()


def plan(M, kPerRank, rank_size, N, commMSize, buffer_count, num_cus=256, opts=None) -> Plan:
    """The plan create() would choose, computed on the host only."""
    p = Plan()
    check(load().mxgemm_seg_plan(ctypes.byref(p), M, kPerRank, rank_size, N, commMSize,
                                 buffer_count, num_cus,
                                 ctypes.byref(opts) if opts is not None else None))
    return p


def decode(p: Plan, rows: int, w: int, block: int):
    tm, tn, ks, fw = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    check(load().mxgemm_seg_decode(ctypes.byref(p), rows, w, block, ctypes.byref(tm),
                                   ctypes.byref(tn), ctypes.byref(ks), ctypes.byref(fw)))
    return tm.value, tn.value, ks.value, fw.value


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dptr(t):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


class SegGemm:
    """Handle for one segmented-GEMM problem shape (mxgemm_seg_create)."""

    def __init__(self, M, kPerRank, rank_size, N, commMSize, buffer_count, opts=None):
        lib = load()
        h = ctypes.c_void_p()
        if opts is None:
            rc = lib.mxgemm_seg_create(ctypes.byref(h), M, kPerRank, rank_size, N, commMSize,
                                       buffer_count)
        else:
            rc = lib.mxgemm_seg_create_ex(ctypes.byref(h), M, kPerRank, rank_size, N, commMSize,
                                          buffer_count, ctypes.byref(opts))
        check(rc)
        self._h = h
        self.M, self.kPerRank, self.R, self.N = M, kPerRank, rank_size, N
        self.K = rank_size * kPerRank

    @property
    def plan(self) -> Plan:
        p = Plan()
        check(load().mxgemm_seg_get_plan(self._h, ctypes.byref(p)))
        return p

    def run(self, a_seg, a_scale, b, b_scale, c, stream=None):
        """Enqueue C = segmented MXFP8 GEMM on `stream` (torch tensors:
        uint8 a_seg [R,M,kPerRank], a_scale [R,M,kPerRank/32], b [N,K],
        b_scale [N,K/32]; bfloat16 c [M,N])."""
        import torch
        exp = {"a_seg": (a_seg, (self.R, self.M, self.kPerRank), torch.uint8),
               "a_scale": (a_scale, (self.R, self.M, self.kPerRank // 32), torch.uint8),
               "b": (b, (self.N, self.K), torch.uint8),
               "b_scale": (b_scale, (self.N, self.K // 32), torch.uint8),
               "c": (c, (self.M, self.N), torch.bfloat16)}
        for name, (t, shape, dt) in exp.items():
            if tuple(t.shape) != shape or t.dtype != dt:
                raise ValueError(f"{name}: expected {dt} {shape}, got {t.dtype} {tuple(t.shape)}")
        check(load().mxgemm_seg_run(self._h, _dptr(a_seg), _dptr(a_scale), _dptr(b),
                                    _dptr(b_scale), _dptr(c), _stream_ptr(stream)))

    def run_ptrs(self, a_seg, a_scale, b, b_scale, c, stream_handle):
        """Raw-pointer form (integers), for callers that manage memory."""
        check(load().mxgemm_seg_run(self._h, ctypes.c_void_p(a_seg), ctypes.c_void_p(a_scale),
                                    ctypes.c_void_p(b), ctypes.c_void_p(b_scale),
                                    ctypes.c_void_p(c), ctypes.c_void_p(stream_handle)))

    def status(self):
        """Raise MxgemmError(ETIMEOUT) if a device wait of the flags
        protocol gave up since the last call (waits for the device)."""
        check(load().mxgemm_seg_status(self._h))

    def set_profiling(self, enable: bool):
        check(load().mxgemm_seg_set_profiling(self._h, 1 if enable else 0))

    def kernel_times(self):
        g, s = ctypes.c_double(), ctypes.c_double()
        gn, sn = ctypes.c_int32(), ctypes.c_int32()
        check(load().mxgemm_seg_kernel_times(self._h, ctypes.byref(g), ctypes.byref(gn),
                                             ctypes.byref(s), ctypes.byref(sn)))
        return {"gemm_ms": g.value, "gemm_launches": gn.value,
                "stage_ms": s.value, "stage_launches": sn.value}

    def close(self):
        if getattr(self, "_h", None):
            rc = load().mxgemm_seg_destroy(self._h)
            self._h = None
            check(rc)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            if getattr(self, "_h", None):
                load().mxgemm_seg_destroy(self._h)
                self._h = None
        except Exception:
            pass


def run_static(M, kPerRank, rank_size, N, commMSize, buffer_count, a_seg, a_scale, b, b_scale, c,
               opts=None, stream=None):
    """mxgemm_seg_run_static: one segmented GEMM with the library's static
    scratch array instead of a handle (allocates nothing).  Tensors as for
    SegGemm.run."""
    import torch
    K = rank_size * kPerRank
    exp = {"a_seg": (a_seg, (rank_size, M, kPerRank), torch.uint8),
           "a_scale": (a_scale, (rank_size, M, kPerRank // 32), torch.uint8),
           "b": (b, (N, K), torch.uint8), "b_scale": (b_scale, (N, K // 32), torch.uint8),
           "c": (c, (M, N), torch.bfloat16)}
    for name, (t, shape, dt) in exp.items():
        if tuple(t.shape) != shape or t.dtype != dt:
            raise ValueError(f"{name}: expected {dt} {shape}, got {t.dtype} {tuple(t.shape)}")
    check(load().mxgemm_seg_run_static(M, kPerRank, rank_size, N, commMSize, buffer_count,
                                       ctypes.byref(opts) if opts is not None else None,
                                       _dptr(a_seg), _dptr(a_scale), _dptr(b), _dptr(b_scale),
                                       _dptr(c), _stream_ptr(stream)))


def quantize_mxfp8(x, q=None, s=None, stream=None, fmt=FMT_E4M3):
    """GPU MXFP8 quantiser: float32 device tensor [rows, cols] (cols % 32 == 0,
    last dim contiguous) -> (uint8 codes [rows, cols] of format ``fmt``,
    uint8 scales [rows, cols/32]).  Outputs may be given (views with unit
    last stride)."""
    import torch
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise TypeError("x must be a device tensor")
    if x.dtype != torch.float32 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D float32 tensor with contiguous rows")
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    for t in (q, s):
        if not isinstance(t, torch.Tensor) or t.device != x.device or t.dtype != torch.uint8:
            raise TypeError("outputs must be uint8 tensors on x's device")
    if q.stride(1) != 1 or s.stride(1) != 1 or tuple(q.shape) != (rows, cols) \
            or tuple(s.shape) != (rows, cols // 32):
        raise ValueError("bad output tensors")
    check(load().mxgemm_quantize_mx(ctypes.c_void_p(x.data_ptr()), rows, cols, x.stride(0),
                                    ctypes.c_void_p(q.data_ptr()), q.stride(0),
                                    ctypes.c_void_p(s.data_ptr()), s.stride(0),
                                    max(0, _fmt(fmt)), _stream_ptr(stream)))
    return q, s


def quantize_segments(a32, R: int, stream=None, fmt=FMT_E4M3):
    """Quantise float32 A [M, K] straight into the segment layout:
    codes [R, M, K/R] and scales [R, M, K/(32R)] (one quantiser launch per
    segment, each reading a column slice of A)."""
    import torch
    M, K = a32.shape
    kpr = K // R
    q = torch.empty((R, M, kpr), dtype=torch.uint8, device=a32.device)
    s = torch.empty((R, M, kpr // 32), dtype=torch.uint8, device=a32.device)
    for r in range(R):
        quantize_mxfp8(a32[:, r * kpr:(r + 1) * kpr], q[r], s[r], stream=stream, fmt=fmt)
    return q, s
