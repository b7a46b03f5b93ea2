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

// E8M0 scale byte b (the low byte of s) -> the float multiplier of its
// block for the scaled bfloat16 conversion, in two instructions (byte
// extract, shift-or): the bits (b << 23) | b.  For b in 1..254 that is
// 2^(b - 127) * (1 + b * 2^-23); the conversion rounds code * multiplier to
// bfloat16, and a code has at most four significant bits, so a relative
// excess below 2^-15 never changes the rounded value: the result is exactly
// code * 2^(b - 127) (as long as that is on the bfloat16 grid, scale byte
// >= 3 for E4M3 codes, >= 10 for E5M2).  b = 0xFF gives a NaN (exponent all
// ones, mantissa nonzero), so every product of its block, zero codes
// included, is NaN; b = 0 gives +0, so a block whose scale is 2^-127
// contributes 0 instead of values below 2^-118.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s)
{
    const uint32_t b = s & 0xFFu;
    return __uint_as_float((b << 23) | b);
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

// The same copies, from a wave-uniform base plus a 32-bit per-lane byte
// offset, issued as inline assembly (global_load_lds_dwordx4 / _dword with
// the SGPR-base address form).  Once the compiler has issued an LDS DMA
// itself, every later wait for an LDS read becomes lgkmcnt(0): it waits for
// all reads in flight, including those issued sub-steps ahead, which undoes
// the GEMM kernels' read-ahead (measured: 225 vs 231 us per 2048 x 8192 x
// 8192 exact launch, 103 vs 106 us per 2048 x 4096 x 7168 one).  Hidden
// from the compiler, the copies need explicit ordering, which the GEMM
// kernels have anyway: a stage is read only after `s_waitcnt vmcnt` and a
// barrier, and written only after a barrier that ends its reads.  The
// instruction has no result registers (it writes LDS), and its address
// registers are read at issue, as for the compiler's own loads.  M0 (the
// LDS destination) is set by the compiler through the "{m0}" operand; the
// s_nop gives the wait states an M0 or SGPR write needs before a vector
// memory instruction reads it.  Extra loads the compiler does not know of
// only make its own vmcnt waits stricter, never shorter (vector memory
// loads return in order).
__device__ __forceinline__ uint32_t lds_addr(void* lds)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
}
__device__ __forceinline__ void dma16_at(const void* base, uint32_t off, void* lds)
{
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_addr(lds)));
}
__device__ __forceinline__ void dma4_at(const void* base, uint32_t off, void* lds)
{
    asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_addr(lds)));
}

typedef float v16f __attribute__((ext_vector_type(16)));

// ---- data one work-group writes for another in the same launch ----------
// Each XCD has its own L2, so such data is written with device-scope stores
// (SC1: written through to the memory side) and read with device-scope
// loads (SC1: a stale L2 line is not used), and a counter is raised only
// once the writer's stores have completed (stores_done).  This avoids the
// agent-wide release / acquire fences, which write back or invalidate a
// whole L2.

// 4-byte device-scope store (a relaxed agent-scope atomic store).
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p)
{
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte device-scope store (global_store_dwordx4 with SC1; its data is
// read at issue).  The compiler does not count it: stores_done() waits.
__device__ __forceinline__ void st_dev16(void* p, const u32x4& v)
{
    asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}

// Eight 16-byte device-scope loads and the wait for them in one statement,
// so no use of a result can be placed before the data has arrived.
__device__ __forceinline__ void ld_dev16x8(const void* const (&p)[8], u32x4 (&v)[8])
{
    asm volatile(
        "global_load_dwordx4 %0, %8, off sc1\n\t"
        "global_load_dwordx4 %1, %9, off sc1\n\t"
        "global_load_dwordx4 %2, %10, off sc1\n\t"
        "global_load_dwordx4 %3, %11, off sc1\n\t"
        "global_load_dwordx4 %4, %12, off sc1\n\t"
        "global_load_dwordx4 %5, %13, off sc1\n\t"
        "global_load_dwordx4 %6, %14, off sc1\n\t"
        "global_load_dwordx4 %7, %15, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
          "=&v"(v[6]), "=&v"(v[7])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7])
        : "memory");
}

// Until this thread's stores (and atomics) have completed.
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Split-K combine of one tile by one work-group: for the tile's valid rows
// r < nrows and columns col0 + cc < N (cc < tile_n),
//   c[(row0 + r) N + col0 + cc] = bf16(sum over t = 0 .. split - 1, in order,
//                                      of ws[t plane + (row0 + r) N + col0 + cc]),
// the partials read with device-scope loads, eight splits at a time, four
// columns per thread.
__device__ inline void combine_tile(const float* ws, int64_t plane, uint16_t* c, int64_t row0,
                                    int nrows, int col0, int tile_n, int N, int split, bool c_vec4)
{
    for (int e = threadIdx.x * 4; e < nrows * tile_n; e += blockDim.x * 4) {
        const int r = e / tile_n, cc = e - r * tile_n;
        const int col = col0 + cc;
        if (col >= N)
            continue;
        const int64_t idx = (row0 + r) * N + col;
        const int nv = (N & 3) == 0 ? 4 : (N - col < 4 ? N - col : 4);
        v4f sum = v4f{0.f, 0.f, 0.f, 0.f};
        for (int t0 = 0; t0 < split; t0 += 8) {
            v4f part[8];
            if (nv == 4 && (N & 3) == 0) {
                // splits past the last read split 0 again (ignored)
                const void* src[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    src[i] = ws + (t0 + i < split ? (int64_t)(t0 + i) * plane : 0) + idx;
                u32x4 raw[8];
                ld_dev16x8(src, raw);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    part[i] = __builtin_bit_cast(v4f, raw[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    part[i] = v4f{0.f, 0.f, 0.f, 0.f};
                    if (t0 + i < split)
                        for (int v = 0; v < nv; ++v)
                            part[i][v] = ld_dev(ws + (int64_t)(t0 + i) * plane + idx + v);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (t0 + i < split) {
                    if (t0 + i == 0) {
                        sum = part[i];
                    } else {
                        sum[0] += part[i][0];
                        sum[1] += part[i][1];
                        sum[2] += part[i][2];
                        sum[3] += part[i][3];
                    }
                }
        }
        if (nv == 4 && c_vec4) {
            *reinterpret_cast<u32x2*>(c + idx) = u32x2{pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])};
        } else {
            for (int v = 0; v < nv; ++v)
                c[idx + v] = f32_to_bf16_rne(sum[v]);
        }
    }
}

template <int MW>
struct AccT;
template <>
struct AccT<16> { typedef v4f T; static constexpr int N = 4; };
template <>
struct AccT<32> { typedef v16f T; static constexpr int N = 16; };

}  // namespace mxg
