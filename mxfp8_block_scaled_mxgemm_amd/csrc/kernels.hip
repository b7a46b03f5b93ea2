// gfx950 kernels of the segmented MXFP8 GEMM: segment staging, the split-K
// reduction, the MXFP8 quantiser, the tile table, and the dispatch to the
// GEMM kernels (gemm_impl.h, one translation unit per FP8 format pair).
#include "device_util.h"
#include "schedule.h"

namespace mxg {

// ----------------------------------------------------------------- table --

// LDS of a work-group: two stages of CH K-steps
template <int BM, int BN, int CH>
constexpr int lds_bytes_for()
{
    return 2 * CH * (BM * kBK + BN * kBK + 4 * (BM > 64 ? BM : 64) + 4 * (BN > 64 ? BN : 64));
}

static const TileCfg kCfgs[] = {
    // rel_rate: planner's throughput per CU relative to the 256x256 tile
    // (threads: exact form; the native 256x256 form runs 512).  The
    // 256x256 tile is native only: its exact form's running and fresh FP32
    // accumulators (128 x 128 outputs per wave, twice) would not fit the
    // register file.
    {256, 256, 512, lds_bytes_for<256, 256, 1>(), 1, 1.00f, 1, false, true, 1, true},
    // 256 x 128: exact on eight waves (two 64 x 64 wave tiles per SIMD, so
    // one wave's accumulator flush overlaps the other's MFMAs; measured 248
    // vs 261 us per 2048 x 8192 x 8192 launch with four 128 x 64 waves)
    {256, 128, 512, lds_bytes_for<256, 128, 1>(), 1, 0.89f, 1, true, true, 1, true},
    {128, 128, 256, lds_bytes_for<128, 128, 1>(), 1, 0.53f, 1, true, true, 1, true},
    {64, 64, 256, lds_bytes_for<64, 64, 2>(), 2, 0.30f, 2, true, true, 1, true},
    {32, 64, 256, lds_bytes_for<32, 64, 3>(), 2, 0.20f, 3, true, true, 1, true},
    {16, 64, 256, lds_bytes_for<16, 64, 3>(), 2, 0.12f, 3, true, true, 1, true},
    // one stage holding a work item's whole K range (at most kOneShotSteps);
    // measured slower than the pipelined tiles wherever it fits
    {32, 64, 256, lds_bytes_for<32, 64, kOneShotSteps>() / 2, 1, 0.20f, kOneShotSteps, true, false, 1, true},
    // 64 x 64 with four K groups of one 64 x 64 wave each (a stage holds one
    // K-step per group); exact mode measured 52.4 vs 62.8 us per run of
    // 1024 x 2048 x 4096 (4 ranks) against 64 x 64 tiles with S = 2
    {64, 64, 256, lds_bytes_for<64, 64, 4>(), 1, 0.60f, 4, true, true, 4, true},
};

int num_tile_cfgs() { return (int)(sizeof(kCfgs) / sizeof(kCfgs[0])); }
const TileCfg& tile_cfg(int i) { return kCfgs[i]; }

// --------------------------------------------------------------- staging --

// blockIdx.y enumerates (chunk, segment) pairs, data pairs first, then
// scale pairs; blockIdx.x strides over the pair's contiguous bytes.  Each
// pair is one contiguous source block -> one contiguous ring block
// (all_to_all_comm_udma.h, PutSegmentToRank: source offset
// r*M*rowBytes + mOffset*rowBytes, destination slot r of the buffer).
__global__ void __launch_bounds__(256) stage_kernel(StageArgs p)
{
    int pair = blockIdx.y;
    const int npairs = p.nch * p.R;
    const bool is_scale = pair >= npairs;
    if (is_scale)
        pair -= npairs;
    const int cidx = pair / p.R;
    const int r = pair - cidx * p.R;
    const int64_t j = p.chunk0 + cidx;
    const int64_t slot = j & (p.nbuf - 1);
    // rows of chunk j: commMSize, or what is left of M for the last chunk
    const int64_t left = p.M - j * p.cms;
    const int64_t nrows = left < p.cms ? left : p.cms;
    if (!is_scale) {
        const int64_t len16 = (nrows * p.kpr) >> 4;
        const u32x4* src = reinterpret_cast<const u32x4*>(p.a_seg + (r * p.M + j * p.cms) * p.kpr);
        u32x4* dst = reinterpret_cast<u32x4*>(p.ring + slot * p.slot_bytes + r * p.cms * p.kpr);
        const int64_t stride = (int64_t)gridDim.x * blockDim.x;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < len16; i += stride)
            dst[i] = __builtin_nontemporal_load(src + i);
    } else {
        const int64_t sk = p.kpr >> 5;
        const int64_t len4 = (nrows * sk) >> 2;
        const uint32_t* src =
            reinterpret_cast<const uint32_t*>(p.sa_seg + (r * p.M + j * p.cms) * sk);
        uint32_t* dst =
            reinterpret_cast<uint32_t*>(p.sring + slot * p.scale_slot_bytes + r * p.cms * sk);
        const int64_t stride = (int64_t)gridDim.x * blockDim.x;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < len4; i += stride)
            dst[i] = src[i];
    }
}

hipError_t launch_stage(const StageArgs& a, hipStream_t stream)
{
    const int64_t len16 = (a.cms * a.kpr) >> 4;
    int64_t bx = (len16 + 256 * 4 - 1) / (256 * 4);
    if (bx < 1)
        bx = 1;
    if (bx > 1024)
        bx = 1024;
    dim3 grid((unsigned)bx, (unsigned)(2 * a.nch * a.R));
    hipLaunchKernelGGL(stage_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

// Split-K reduction: four consecutive outputs per thread; the splits are
// summed in index order, so the result does not depend on timing.
__global__ void __launch_bounds__(256) reduce_kernel(ReduceArgs p)
{
    const int64_t total = (int64_t)p.rows * p.N;
    const int64_t slice = total;
    const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i4 >= total)
        return;
    if ((p.N & 3) == 0) {
        v4f s = *reinterpret_cast<const v4f*>(p.ws + i4);
        for (int k = 1; k < p.split; ++k) {
            const v4f t = *reinterpret_cast<const v4f*>(p.ws + (int64_t)k * slice + i4);
            s[0] += t[0];
            s[1] += t[1];
            s[2] += t[2];
            s[3] += t[3];
        }
        if (p.c_vec4) {
            *reinterpret_cast<u32x2*>(p.c + i4) = u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                p.c[i4 + u] = f32_to_bf16_rne(s[u]);
        }
        return;
    }
    for (int64_t e = i4; e < i4 + 4 && e < total; ++e) {
        float s = p.ws[e];
        for (int k = 1; k < p.split; ++k)
            s += p.ws[(int64_t)k * slice + e];
        p.c[e] = f32_to_bf16_rne(s);
    }
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream)
{
    const int64_t threads = ((int64_t)a.rows * a.N + 3) / 4;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// Fill n 32-bit words with v (a kernel, not a memset, so the call can sit
// in a captured HIP graph).
__global__ void __launch_bounds__(256) fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t stream)
{
    if (n <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n, v);
    return hipGetLastError();
}

// -------------------------------------------------------- GEMM dispatch --

template <int FA, int FB>
hipError_t launch_gemm_fmt(int cfg, bool exact, const GemmArgs& a, hipStream_t stream);
extern template hipError_t launch_gemm_fmt<kE4M3, kE4M3>(int, bool, const GemmArgs&, hipStream_t);
extern template hipError_t launch_gemm_fmt<kE5M2, kE5M2>(int, bool, const GemmArgs&, hipStream_t);
extern template hipError_t launch_gemm_fmt<kE4M3, kE5M2>(int, bool, const GemmArgs&, hipStream_t);
extern template hipError_t launch_gemm_fmt<kE5M2, kE4M3>(int, bool, const GemmArgs&, hipStream_t);

hipError_t launch_gemm(int cfg, bool exact, int fa, int fb, const GemmArgs& a, hipStream_t stream)
{
    if (fa == kE4M3 && fb == kE4M3)
        return launch_gemm_fmt<kE4M3, kE4M3>(cfg, exact, a, stream);
    if (fa == kE5M2 && fb == kE5M2)
        return launch_gemm_fmt<kE5M2, kE5M2>(cfg, exact, a, stream);
    if (fa == kE4M3 && fb == kE5M2)
        return launch_gemm_fmt<kE4M3, kE5M2>(cfg, exact, a, stream);
    if (fa == kE5M2 && fb == kE4M3)
        return launch_gemm_fmt<kE5M2, kE4M3>(cfg, exact, a, stream);
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------- quantiser --

// E4M3 (OCP "FN") code of a non-NaN float, round-to-nearest-even, sign of
// zero kept; magnitudes above 448 after rounding (infinities included)
// saturate to 448 (code 0x7E).  Normal range: keep 3 mantissa bits and
// round on the 20 dropped bits; below 2^-6 the grid step is 2^-9, so
// y * 512 rounded to an integer is the code (8 is the smallest normal,
// code 0x08).
__device__ __forceinline__ uint32_t e4m3_rne(float y)
{
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a < 0x3C800000u) {                       // |y| < 2^-6
        code = (uint32_t)rintf(__uint_as_float(a) * 512.0f);
    } else {
        const uint32_t keep = (a >> 20) & 7u;
        const uint32_t rest = a & 0xFFFFFu;
        code = (((a >> 23) - 120u) << 3) | keep;  // biased exponent 127 -> 7
        if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u)))
            code += 1u;
        if (code > 0x7Eu)
            code = 0x7Eu;
    }
    return code | sign;
}

// E5M2 (OCP, bias 15) code of a float, round-to-nearest-even, saturating at
// the largest finite value 57344 (code 0x7B) instead of producing infinity.
// Normal range: keep 2 mantissa bits and round on the 21 dropped bits;
// below 2^-14 the grid step is 2^-16, so y * 65536 rounded to an integer is
// the code (4 is the smallest normal, code 0x04).
__device__ __forceinline__ uint32_t e5m2_rne(float y)
{
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a < 0x38800000u) {                       // |y| < 2^-14
        code = (uint32_t)rintf(__uint_as_float(a) * 65536.0f);
    } else {
        const uint32_t keep = (a >> 21) & 3u;
        const uint32_t rest = a & 0x1FFFFFu;
        code = (((a >> 23) - 112u) << 2) | keep;  // biased exponent 127 -> 15
        if (rest > 0x100000u || (rest == 0x100000u && (keep & 1u)))
            code += 1u;
        if (code > 0x7Bu)
            code = 0x7Bu;
    }
    return code | sign;
}

// Smallest e with fmax * 2^e >= amax, clamped to [-127, 127], for the
// format's largest finite value fmax = 1.75 * 2^EMAX (448: EMAX = 8 for
// E4M3; 57344: EMAX = 15 for E5M2).  With amax = 1.m * 2^x, e = x - EMAX
// when 1.m <= 1.75, else x - EMAX + 1.  Zero and float32 subnormals give
// -127 (the clamp), +inf gives 127 (the clamp of an unbounded e); amax is
// never NaN here (NaN blocks are handled by the caller).
template <int EMAX>
__device__ __forceinline__ int e8m0_exponent(float amax)
{
    const uint32_t u = __float_as_uint(amax);
    const int ex = (int)(u >> 23);
    if (ex == 0)
        return -127;
    if (ex == 255)
        return 127;
    int e = ex - 127 - EMAX + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    e = e < -127 ? -127 : e;
    return e > 127 ? 127 : e;
}

template <int F>
__device__ __forceinline__ uint32_t fp8_rne(float y)
{
    return F == kE5M2 ? e5m2_rne(y) : e4m3_rne(y);
}

// Eight threads per 32-element block, four elements each.  The block's
// amax is the largest |x| bit pattern: for non-negative floats the integer
// order is the numeric order, and every NaN pattern lies above +inf
// (0x7F800000), so a NaN anywhere in the block is seen (a float max would
// drop it).  A NaN block has no exponent: scale byte 0xFF (the E8M0 NaN)
// and every code the NaN code 0x7F.  Infinities (with no NaN) give e = 127
// and saturate to the largest finite code of their sign.
template <int F>
__global__ void __launch_bounds__(256) quantize_kernel(QuantArgs p)
{
    const int64_t nblk_row = p.cols >> 5;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t blk = gid >> 3;
    const int part = (int)(gid & 7);
    const bool valid = blk < p.rows * nblk_row;
    const int64_t row = valid ? blk / nblk_row : 0;
    const int64_t cb = valid ? blk - row * nblk_row : 0;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid)
        v = *reinterpret_cast<const float4*>(p.x + row * p.ld_x + cb * 32 + part * 4);
    const uint32_t am = 0x7FFFFFFFu;
    uint32_t m = max(max(__float_as_uint(v.x) & am, __float_as_uint(v.y) & am),
                     max(__float_as_uint(v.z) & am, __float_as_uint(v.w) & am));
    m = max(m, (uint32_t)__shfl_xor((int)m, 1, 8));
    m = max(m, (uint32_t)__shfl_xor((int)m, 2, 8));
    m = max(m, (uint32_t)__shfl_xor((int)m, 4, 8));
    if (!valid)
        return;
    uint32_t code;
    uint8_t sbyte;
    if (m > 0x7F800000u) {
        code = 0x7F7F7F7Fu;
        sbyte = 0xFF;
    } else {
        const int e = e8m0_exponent<F == kE5M2 ? 15 : 8>(__uint_as_float(m));
        code = fp8_rne<F>(ldexpf(v.x, -e)) | (fp8_rne<F>(ldexpf(v.y, -e)) << 8) |
               (fp8_rne<F>(ldexpf(v.z, -e)) << 16) | (fp8_rne<F>(ldexpf(v.w, -e)) << 24);
        sbyte = (uint8_t)(e + 127);
    }
    *reinterpret_cast<uint32_t*>(p.q + row * p.ld_q + cb * 32 + part * 4) = code;
    if (part == 0)
        p.s[row * p.ld_s + cb] = sbyte;
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream)
{
    const int64_t threads = a.rows * (a.cols >> 5) * 8;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks == 0)
        return hipSuccess;
    if (a.fmt == kE5M2)
        hipLaunchKernelGGL(quantize_kernel<kE5M2>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(quantize_kernel<kE4M3>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mxg
