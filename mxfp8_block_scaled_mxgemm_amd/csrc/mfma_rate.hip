// MFMA throughput probe for the benchmark's measured denominator: every
// wave issues back-to-back MFMAs on four independent accumulators, with no
// memory traffic inside the loop, so the launch runs at the matrix cores'
// sustained rate (at whatever clock the part holds under that load).  Not
// part of the GEMM library; bench.py loads it on its own.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// kind 0: v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 codes (131072 FLOP each);
// kind 1: v_mfma_f32_32x32x16_bf16 (32768 FLOP each).
template <int KIND>
__global__ void __launch_bounds__(256) mfma_rate_kernel(float* out, int iters)
{
    // E4M3 1.0 (0x38) in every byte; bfloat16 1.0 (0x3F80) in every half
    const int lane_bits = (int)(threadIdx.x & 1);
    v8i a8, b8;
    for (int i = 0; i < 8; ++i) {
        a8[i] = 0x38383838 ^ lane_bits;
        b8[i] = 0x38383838;
    }
    v8bf a16, b16;
    for (int i = 0; i < 8; ++i) {
        a16[i] = (__bf16)1.0f;
        b16[i] = (__bf16)(lane_bits ? 0.5f : 1.0f);
    }
    v16f acc[4];
    for (int j = 0; j < 4; ++j)
        for (int v = 0; v < 16; ++v)
            acc[j][v] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (KIND == 0)
                    acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[j], 0, 0, 0, 127,
                                                                             0, 127);
                else
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a16, b16, acc[j], 0, 0, 0);
            }
    }
    float s = 0.f;
    for (int j = 0; j < 4; ++j)
        for (int v = 0; v < 16; ++v)
            s += acc[j][v];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// Launch `grid` work-groups of 256 threads; each wave issues iters * 16
// MFMAs of the given kind.  out holds grid * 256 floats.  Returns 0 or the
// HIP error code.
extern "C" int mxgemm_probe_mfma_rate(int kind, int grid, int iters, float* out, void* stream)
{
    if (grid <= 0 || iters <= 0 || !out || (kind != 0 && kind != 1))
        return (int)hipErrorInvalidValue;
    if (kind == 0)
        hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(grid), dim3(256), 0, (hipStream_t)stream, out, iters);
    else
        hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(grid), dim3(256), 0, (hipStream_t)stream, out, iters);
    return (int)hipGetLastError();
}
