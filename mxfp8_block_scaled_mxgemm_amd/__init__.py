"""Segmented MXFP8 GEMM for AMD Instinct MI355X (gfx950).

The compute half of a fused all-to-all + MXFP8 matmul: R simulated ranks'
A segments are staged chunk by chunk into a ring of buffers and consumed by
a block-scaled FP8 GEMM on CDNA4 scaled MFMA, producing bfloat16 C.  The
work runs in the HIP library ``libmxgemm_seg.so`` behind the C ABI in
``include/mxgemm_seg.h``; this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    EXPORTED, FMT_E4M3, FMT_E5M2, PRECISION_EXACT, PRECISION_NATIVE, RING_EVENTS, RING_FLAGS,
    MxgemmError, Options, Plan, SegGemm, decode,
    last_error, load, options, plan, quantize_mxfp8, quantize_segments, run_static,
)
