// gfx950 kernels of the segmented MXFP8 GEMM: segment staging, the
// block-scaled GEMM on CDNA4 scaled FP8 MFMA, and the MXFP8 quantiser.
#include "kernels.h"
#include "schedule.h"

namespace mxg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------- table --

// MFMA K-step: one v_mfma_scale_f32_16x16x128_f8f6f4 consumes 128 K per
// row, i.e. four 32-element MX blocks.  Operand layout (measured with a
// one-wave probe of the builtin): lane l holds row (or column) l % 16; with
// q = l / 16 its 32 bytes are K [16q, 16q + 16) followed by K
// [64 + 16q, 64 + 16q + 16), and its scale byte applies to MX block q, i.e.
// K [32q, 32q + 32).  The result is D[4 * (l / 16) + v][l % 16] in
// accumulator element v.
constexpr int kBK = 128;

template <int BM, int BN>
constexpr int lds_bytes_for() { return 2 * (BM * kBK + BN * kBK + 4 * BM + 4 * BN); }

static const TileCfg kCfgs[] = {
    {256, 128, 256, lds_bytes_for<256, 128>(), 1, 0.90f},
    {128, 128, 256, lds_bytes_for<128, 128>(), 1, 0.75f},
    {64, 64, 256, lds_bytes_for<64, 64>(), 4, 0.45f},
    {32, 64, 256, lds_bytes_for<32, 64>(), 4, 0.30f},
    {16, 64, 256, lds_bytes_for<16, 64>(), 4, 0.20f},
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
    if (!is_scale) {
        const int64_t len16 = (p.cms * p.kpr) >> 4;
        const u32x4* src = reinterpret_cast<const u32x4*>(p.a_seg + (r * p.M + j * p.cms) * p.kpr);
        u32x4* dst = reinterpret_cast<u32x4*>(p.ring + slot * p.slot_bytes + r * p.cms * p.kpr);
        const int64_t stride = (int64_t)gridDim.x * blockDim.x;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < len16; i += stride)
            dst[i] = __builtin_nontemporal_load(src + i);
    } else {
        const int64_t sk = p.kpr >> 5;
        const int64_t len4 = (p.cms * sk) >> 2;
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

// ------------------------------------------------------------------ GEMM --

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// E8M0 scale byte -> 2^(s - 127) as float (s = 0 is the float32 subnormal
// 2^-127; 0xFF is NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s)
{
    s &= 0xFFu;
    if (s == 0xFFu)
        return __uint_as_float(0x7FC00000u);
    return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);
}

// Eight E4M3 codes -> eight bfloat16 values times `scale`, in order.
__device__ __forceinline__ v8bf fp8x8_to_bf16(u32x2 raw, float scale)
{
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, scale, false);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, scale, true);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, scale, false);
    const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, scale, true);
    return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// LDS tile rows are kBK = 128 bytes = eight 16-byte chunks.  The chunk
// position is XOR-swizzled with the row so that the 16 lanes reading the
// same K chunk of 16 consecutive rows hit different banks.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

template <int BM, int BN, int WGM, int WGN, int OCC, bool EXACT>
__global__ void __launch_bounds__(WGM * WGN * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
mxgemm_kernel(GemmArgs p)
{
    constexpr int NT = WGM * WGN * 64;
    constexpr int TM = BM / WGM, TN = BN / WGN;
    constexpr int GA = TM / 16, GB = TN / 16;
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
    constexpr int A_BYTES = BM * kBK, B_BYTES = BN * kBK;
    constexpr int STAGE = A_BYTES + B_BYTES + 4 * BM + 4 * BN;
    constexpr int CA = (BM * 8 + NT - 1) / NT;   // 16-byte A chunks per thread
    constexpr int CB = (BN * 8 + NT - 1) / NT;
    constexpr int SA = (BM + NT - 1) / NT;       // A scale dwords per thread
    constexpr int SB = (BN + NT - 1) / NT;
    constexpr bool A_FULL = (BM * 8) % NT == 0, B_FULL = (BN * 8) % NT == 0;

    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int l16 = lane & 15, kb = lane >> 4;

    const int steps_per_seg = p.kpr / kBK;
    const int sk = p.kpr >> 5;              // scale bytes per row per segment
    const int K32 = p.K >> 5;

    for (int w = remap_block(blockIdx.x, gridDim.x); w < p.total_work; w += gridDim.x) {
        const TileCoord tc = decode_work(w, p.tiles_m, p.tiles_n, p.split, p.group_n);
        const int m0 = tc.tm * BM, n0 = tc.tn * BN;

        // Per-thread 32-bit row offsets for this tile.  A offsets are
        // relative to the window's ring base (the ring is < 2 GiB), B
        // offsets relative to row n0 of B.  Rows past the edge are clamped
        // to the last valid row; their results are never stored.
        uint32_t a_off[CA], b_off[CB], as_off[SA], bs_off[SB];
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int idx = tid + i * NT;
            const int row = (idx >> 3) < BM ? (idx >> 3) : BM - 1, ch = idx & 7;
            int g = m0 + row;
            g = g < p.rows ? g : p.rows - 1;
            a_off[i] = (uint32_t)((g / p.cms) * p.a_slot_stride) + (uint32_t)((g % p.cms) * p.kpr) + ch * 16;
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int idx = tid + i * NT;
            const int row = (idx >> 3) < BN ? (idx >> 3) : BN - 1, ch = idx & 7;
            int g = row;
            g = n0 + g < p.N ? g : p.N - 1 - n0;
            b_off[i] = (uint32_t)g * (uint32_t)p.K + ch * 16;
        }
#pragma unroll
        for (int i = 0; i < SA; ++i) {
            const int row = (tid + i * NT) < BM ? tid + i * NT : BM - 1;
            int g = m0 + row;
            g = g < p.rows ? g : p.rows - 1;
            as_off[i] = (uint32_t)((g / p.cms) * p.as_slot_stride) + (uint32_t)((g % p.cms) * sk);
        }
#pragma unroll
        for (int i = 0; i < SB; ++i) {
            const int row = (tid + i * NT) < BN ? tid + i * NT : BN - 1;
            int g = row;
            g = n0 + g < p.N ? g : p.N - 1 - n0;
            bs_off[i] = (uint32_t)g * (uint32_t)K32;
        }
        const uint8_t* __restrict__ bt = p.b + (int64_t)n0 * p.K;
        const uint8_t* __restrict__ bst = p.bs + (int64_t)n0 * K32;

        const int seg0 = tc.ks * p.segs_per_split;
        const int nsteps = p.segs_per_split * steps_per_seg;

        u32x4 ra[CA], rb[CB];
        uint32_t rsa[SA], rsb[SB];

        v4f acc[GA][GB];
#pragma unroll
        for (int i = 0; i < GA; ++i)
#pragma unroll
            for (int j = 0; j < GB; ++j)
                acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

// global -> registers for K-step S of this split
#define MXG_LOAD_STEP(S)                                                                   \
    do {                                                                                   \
        const int seg_ = seg0 + (S) / steps_per_seg;                                       \
        const int kk_ = ((S) % steps_per_seg) * kBK;                                       \
        const uint8_t* __restrict__ a_ = p.a + (int64_t)seg_ * p.cms * p.kpr + kk_;         \
        const uint8_t* __restrict__ b_ = bt + (int64_t)seg_ * p.kpr + kk_;                  \
        const uint8_t* __restrict__ as_ = p.as + (int64_t)seg_ * p.cms * sk + (kk_ >> 5);   \
        const uint8_t* __restrict__ bs_ = bst + (((int64_t)seg_ * p.kpr + kk_) >> 5);       \
        _Pragma("unroll") for (int i = 0; i < CA; ++i)                                     \
            ra[i] = *reinterpret_cast<const u32x4*>(a_ + a_off[i]);                        \
        _Pragma("unroll") for (int i = 0; i < CB; ++i)                                     \
            rb[i] = *reinterpret_cast<const u32x4*>(b_ + b_off[i]);                        \
        _Pragma("unroll") for (int i = 0; i < SA; ++i)                                     \
            rsa[i] = *reinterpret_cast<const uint32_t*>(as_ + as_off[i]);                  \
        _Pragma("unroll") for (int i = 0; i < SB; ++i)                                     \
            rsb[i] = *reinterpret_cast<const uint32_t*>(bs_ + bs_off[i]);                  \
    } while (0)

// registers -> LDS stage buffer BUF
#define MXG_STORE_STEP(BUF)                                                                \
    do {                                                                                   \
        uint8_t* sa_ = smem + (BUF) * STAGE;                                               \
        uint8_t* sb_ = sa_ + A_BYTES;                                                      \
        uint32_t* ssa_ = reinterpret_cast<uint32_t*>(sb_ + B_BYTES);                       \
        uint32_t* ssb_ = ssa_ + BM;                                                        \
        _Pragma("unroll") for (int i = 0; i < CA; ++i) {                                   \
            const int idx = tid + i * NT;                                                  \
            const int row = idx >> 3, ch = idx & 7;                                        \
            if (A_FULL || idx < BM * 8)                                                    \
                *reinterpret_cast<u32x4*>(sa_ + row * kBK + swz(row, ch) * 16) = ra[i];    \
        }                                                                                  \
        _Pragma("unroll") for (int i = 0; i < CB; ++i) {                                   \
            const int idx = tid + i * NT;                                                  \
            const int row = idx >> 3, ch = idx & 7;                                        \
            if (B_FULL || idx < BN * 8)                                                    \
                *reinterpret_cast<u32x4*>(sb_ + row * kBK + swz(row, ch) * 16) = rb[i];    \
        }                                                                                  \
        _Pragma("unroll") for (int i = 0; i < SA; ++i)                                     \
            if (tid + i * NT < BM)                                                         \
                ssa_[tid + i * NT] = rsa[i];                                               \
        _Pragma("unroll") for (int i = 0; i < SB; ++i)                                     \
            if (tid + i * NT < BN)                                                         \
                ssb_[tid + i * NT] = rsb[i];                                               \
    } while (0)

        __syncthreads();   // the previous work item is done with the LDS
        MXG_LOAD_STEP(0);
        MXG_STORE_STEP(0);
        __syncthreads();

        for (int s = 0; s < nsteps; ++s) {
            const int buf = s & 1;
            if (s + 1 < nsteps)
                MXG_LOAD_STEP(s + 1);

            const uint8_t* sa_ = smem + buf * STAGE;
            const uint8_t* sb_ = sa_ + A_BYTES;
            const uint8_t* ssa = sb_ + B_BYTES;
            const uint8_t* ssb = ssa + 4 * BM;

            if constexpr (!EXACT) {
                v8i bf[GB];
                int sbv[GB];
    #pragma unroll
                for (int j = 0; j < GB; ++j) {
                    const int row = wn * TN + j * 16 + l16;
                    const u32x4 lo = *reinterpret_cast<const u32x4*>(sb_ + row * kBK + swz(row, kb) * 16);
                    const u32x4 hi = *reinterpret_cast<const u32x4*>(sb_ + row * kBK + swz(row, kb + 4) * 16);
                    bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    sbv[j] = ssb[row * 4 + kb];
                }
    #pragma unroll
                for (int i = 0; i < GA; ++i) {
                    const int row = wm * TM + i * 16 + l16;
                    const u32x4 lo = *reinterpret_cast<const u32x4*>(sa_ + row * kBK + swz(row, kb) * 16);
                    const u32x4 hi = *reinterpret_cast<const u32x4*>(sa_ + row * kBK + swz(row, kb + 4) * 16);
                    const v8i af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    const int sav = ssa[row * 4 + kb];
    #pragma unroll
                    for (int j = 0; j < GB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            af, bf[j], acc[i][j], 0 /*A: E4M3*/, 0 /*B: E4M3*/,
                            0, sav, 0, sbv[j]);
                }
            } else {
                // Exact accumulation: each MX block j of the K-step is one
                // v_mfma_f32_16x16x32_bf16.  Lane group q of a 16-row group
                // takes 8 codes of block j (K [32j + 8q, 32j + 8q + 8)),
                // converted to bfloat16 with the block's scale folded in
                // (exact: 4-bit significands times a power of two).  A and
                // B use the same K assignment, so every product pairs
                // correctly; the products are exact in the MFMA and summed
                // with FP32-grade precision.
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int ch = 2 * j + (kb >> 1), half = (kb & 1) * 8;
                    v8bf bb[GB];
#pragma unroll
                    for (int g = 0; g < GB; ++g) {
                        const int row = wn * TN + g * 16 + l16;
                        const u32x2 raw = *reinterpret_cast<const u32x2*>(sb_ + row * kBK + swz(row, ch) * 16 + half);
                        bb[g] = fp8x8_to_bf16(raw, e8m0_to_f32(ssb[row * 4 + j]));
                    }
#pragma unroll
                    for (int i = 0; i < GA; ++i) {
                        const int row = wm * TM + i * 16 + l16;
                        const u32x2 raw = *reinterpret_cast<const u32x2*>(sa_ + row * kBK + swz(row, ch) * 16 + half);
                        const v8bf ab = fp8x8_to_bf16(raw, e8m0_to_f32(ssa[row * 4 + j]));
#pragma unroll
                        for (int g = 0; g < GB; ++g)
                            acc[i][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, bb[g], acc[i][g], 0, 0, 0);
                    }
                }
            }

            if (s + 1 < nsteps)
                MXG_STORE_STEP(buf ^ 1);
            __syncthreads();
        }
#undef MXG_LOAD_STEP
#undef MXG_STORE_STEP

        // ---- epilogue --------------------------------------------------
        const int row_base = m0 + wm * TM + 4 * kb;
        const int col_base = n0 + wn * TN + l16;
        if (p.split == 1) {
#pragma unroll
            for (int i = 0; i < GA; ++i)
#pragma unroll
                for (int j = 0; j < GB; ++j) {
                    const int col = col_base + j * 16;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int row = row_base + i * 16 + v;
                        if (row < p.rows && col < p.N)
                            p.c[(int64_t)row * p.N + col] = f32_to_bf16_rne(acc[i][j][v]);
                    }
                }
        } else {
            // Split-K: every split stores its FP32 partial tile; the last
            // split to arrive sums all partials in split order (so the
            // result does not depend on arrival order) and writes C.
            const int tile_id = tc.tm * p.tiles_n + tc.tn;
            float* wsp = p.ws + ((int64_t)tile_id * p.split + tc.ks) * (BM * BN);
#pragma unroll
            for (int i = 0; i < GA; ++i)
#pragma unroll
                for (int j = 0; j < GB; ++j)
                    *reinterpret_cast<v4f*>(wsp + ((i * GB + j) * NT + tid) * 4) = acc[i][j];
            __threadfence();
            __syncthreads();
            if (tid == 0) {
                const int old = atomicAdd(p.counters + tile_id, 1);
                s_last = (old == p.split - 1);
            }
            __syncthreads();
            if (s_last) {
                __threadfence();
                const float* wst = p.ws + (int64_t)tile_id * p.split * (BM * BN);
#pragma unroll
                for (int i = 0; i < GA; ++i)
#pragma unroll
                    for (int j = 0; j < GB; ++j) {
                        v4f sum = *reinterpret_cast<const v4f*>(wst + ((i * GB + j) * NT + tid) * 4);
                        for (int s = 1; s < p.split; ++s) {
                            const v4f t = *reinterpret_cast<const v4f*>(
                                wst + (int64_t)s * (BM * BN) + ((i * GB + j) * NT + tid) * 4);
                            sum[0] += t[0];
                            sum[1] += t[1];
                            sum[2] += t[2];
                            sum[3] += t[3];
                        }
                        const int col = col_base + j * 16;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int row = row_base + i * 16 + v;
                            if (row < p.rows && col < p.N)
                                p.c[(int64_t)row * p.N + col] = f32_to_bf16_rne(sum[v]);
                        }
                    }
                if (tid == 0)
                    atomicExch(p.counters + tile_id, 0);
            }
        }
    }
}

template <int BM, int BN, int WGM, int WGN, int OCC>
static hipError_t launch_cfg(const GemmArgs& a, int grid, bool exact, hipStream_t stream)
{
    if (exact)
        hipLaunchKernelGGL((mxgemm_kernel<BM, BN, WGM, WGN, OCC, true>), dim3(grid),
                           dim3(WGM * WGN * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((mxgemm_kernel<BM, BN, WGM, WGN, OCC, false>), dim3(grid),
                           dim3(WGM * WGN * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_gemm(int cfg, bool exact, const GemmArgs& a, int grid, hipStream_t stream)
{
    switch (cfg) {
    case 0: return launch_cfg<256, 128, 2, 2, 1>(a, grid, exact, stream);
    case 1: return launch_cfg<128, 128, 2, 2, 1>(a, grid, exact, stream);
    case 2: return launch_cfg<64, 64, 2, 2, 4>(a, grid, exact, stream);
    case 3: return launch_cfg<32, 64, 1, 4, 4>(a, grid, exact, stream);
    case 4: return launch_cfg<16, 64, 1, 4, 4>(a, grid, exact, stream);
    default: return hipErrorInvalidValue;
    }
}

// ------------------------------------------------------------- quantiser --

// E4M3 (OCP "FN") code of a float with |y| <= 448, round-to-nearest-even,
// sign of zero kept.  Normal range: keep 3 mantissa bits and round on the
// 20 dropped bits; below 2^-6 the grid step is 2^-9, so y * 512 rounded to
// an integer is the code (8 is the smallest normal, code 0x08).
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

// Smallest e with 448 * 2^e >= amax, clamped to [-127, 127].  With
// amax = 1.m * 2^x: 448 = 1.75 * 2^8, so e = x - 8 when 1.m <= 1.75, else
// x - 7.  Zero and float32 subnormals give -127 (the clamp).
__device__ __forceinline__ int e8m0_exponent(float amax)
{
    const uint32_t u = __float_as_uint(amax);
    const int ex = (int)(u >> 23);
    if (ex == 0)
        return -127;
    int e = ex - 127 - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    e = e < -127 ? -127 : e;
    return e > 127 ? 127 : e;
}

// Eight threads per 32-element block, four elements each.
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
    float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    m = fmaxf(m, __shfl_xor(m, 1, 8));
    m = fmaxf(m, __shfl_xor(m, 2, 8));
    m = fmaxf(m, __shfl_xor(m, 4, 8));
    if (!valid)
        return;
    const int e = e8m0_exponent(m);
    const uint32_t code = e4m3_rne(ldexpf(v.x, -e)) | (e4m3_rne(ldexpf(v.y, -e)) << 8) |
                          (e4m3_rne(ldexpf(v.z, -e)) << 16) | (e4m3_rne(ldexpf(v.w, -e)) << 24);
    *reinterpret_cast<uint32_t*>(p.q + row * p.ld_q + cb * 32 + part * 4) = code;
    if (part == 0)
        p.s[row * p.ld_s + cb] = (uint8_t)(e + 127);
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream)
{
    const int64_t threads = a.rows * (a.cols >> 5) * 8;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mxg
