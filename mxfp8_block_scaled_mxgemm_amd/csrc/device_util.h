// Device helpers shared by the gfx950 kernels of the segmented MXFP8 GEMM.
#pragma once

#include "kernels.h"

namespace mxg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// FP8 operand formats (the values of MXGEMM_FMT_*)
constexpr int kE4M3 = 0, kE5M2 = 1;

// MFMA K-step: one v_mfma_scale_f32_16x16x128_f8f6f4 consumes 128 K per
// row, i.e. four 32-element MX blocks.  Operand layout (measured with a
// one-wave probe of the builtin): lane l holds row (or column) l % 16; with
// q = l / 16 its 32 bytes are K [16q, 16q + 16) followed by K
// [64 + 16q, 64 + 16q + 16), and its scale byte applies to MX block q, i.e.
// K [32q, 32q + 32).  The result is D[4 * (l / 16) + v][l % 16] in
// accumulator element v.
constexpr int kBK = 128;

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two floats -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32), `lo`
// in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{lo, hi}, v2bf));
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return (uint16_t)pack_bf16x2(f, 0.f); }

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// E8M0 scale byte -> 2^(s - 127) as float, branch-free: v_ldexp_f32 gives
// 2^-127 (a float32 subnormal) for s = 0; the NaN byte 0xFF comes out as
// +inf.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s)
{
    return __builtin_amdgcn_ldexpf(0x1p-127f, (int)(s & 0xFFu));
}

// Two FP8 codes (bytes 2h, 2h + 1 of `src`) of format F -> two bfloat16
// values times `scale` (v_cvt_scalef32_pk_bf16_fp8 / _bf8; exact while the
// product is a multiple of bfloat16's smallest step).
template <int F>
__device__ __forceinline__ uint32_t cvt2(uint32_t src, float scale, bool hi)
{
    if constexpr (F == kE5M2)
        return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(src, scale, true))
                  : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(src, scale, false));
    else
        return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, scale, true))
                  : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, scale, false));
}

// Eight codes of format F -> eight bfloat16 values times `scale`, in order.
template <int F>
__device__ __forceinline__ v8bf fp8x8_to_bf16(u32x2 raw, float scale)
{
    u32x4 r;
    r.x = cvt2<F>(raw.x, scale, false);
    r.y = cvt2<F>(raw.x, scale, true);
    r.z = cvt2<F>(raw.y, scale, false);
    r.w = cvt2<F>(raw.y, scale, true);
    return __builtin_bit_cast(v8bf, r);
}

// LDS tile rows are kBK = 128 bytes = eight 16-byte chunks.  The chunk
// position is XOR-swizzled with the row so that lanes reading the same
// logical chunk of consecutive rows hit different banks.  For 16-row MFMA
// fragments (MW = 16) row & 7 suffices.  With 32-row fragments the lanes of
// rows r and r + 16 are served together, so bit 4 of the row flips the
// chunk as well (measured: 2-way conflicts without it).
template <int MW>
__device__ __forceinline__ int swz_t(int row, int chunk)
{
    return MW == 32 ? chunk ^ (row & 7) ^ ((row >> 4) & 1) : chunk ^ (row & 7);
}
__device__ __forceinline__ int swz(int row, int chunk) { return swz_t<16>(row, chunk); }

// One 16-byte (or 4-byte) piece per lane, straight from global memory into
// LDS at lds + 16 * lane (resp. 4 * lane); lds must be wave-uniform.
__device__ __forceinline__ void dma16(const void* g, void* lds)
{
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds)
{
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

typedef float v16f __attribute__((ext_vector_type(16)));

template <int MW>
struct AccT;
template <>
struct AccT<16> { typedef v4f T; static constexpr int N = 4; };
template <>
struct AccT<32> { typedef v16f T; static constexpr int N = 16; };

}  // namespace mxg
