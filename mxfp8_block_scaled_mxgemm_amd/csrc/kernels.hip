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
constexpr int lds_bytes_for()
{
    return 2 * (BM * kBK + BN * kBK + 4 * (BM > 64 ? BM : 64) + 4 * (BN > 64 ? BN : 64));
}

static const TileCfg kCfgs[] = {
    // rel_rate: measured throughput per CU relative to the 256x256 tile
    {256, 256, 512, lds_bytes_for<256, 256>(), 1, 1.00f},
    {256, 128, 256, lds_bytes_for<256, 128>(), 1, 0.69f},
    {128, 128, 256, lds_bytes_for<128, 128>(), 1, 0.53f},
    {64, 64, 256, lds_bytes_for<64, 64>(), 4, 0.30f},
    {32, 64, 256, lds_bytes_for<32, 64>(), 4, 0.20f},
    {16, 64, 256, lds_bytes_for<16, 64>(), 4, 0.12f},
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

// E8M0 scale byte -> 2^(s - 127) as float, branch-free: v_ldexp_f32 gives
// 2^-127 (a float32 subnormal) for s = 0; the NaN byte 0xFF comes out as
// +inf.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s)
{
    return __builtin_amdgcn_ldexpf(0x1p-127f, (int)(s & 0xFFu));
}

// Eight E4M3 codes -> eight bfloat16 values times `scale`, in order.
__device__ __forceinline__ v8bf fp8x8_to_bf16(u32x2 raw, float scale)
{
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, scale, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, scale, true));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, scale, false));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, scale, true));
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

// Block-scaled GEMM over one window of staged rows.
//
// Work-group tile BM x BN, WGM x WGN waves, K-step 128 (four MX blocks).
// Each K-step's A and B tiles and their scale bytes are copied global ->
// LDS by the load unit itself (global_load_lds), double-buffered, so the
// next step's copy runs while the current one is multiplied and no
// registers hold staged data.  A lane of a copy instruction writes 16 bytes
// at lds_base + 16 * lane: eight lanes fill one 128-byte tile row, and lane
// L fetches the logical chunk that the row's XOR swizzle places at physical
// chunk L % 8.
//
// MW is the MFMA width.  MW = 16: v_mfma_scale_f32_16x16x128_f8f6f4
// (native) or v_mfma_f32_16x16x32_bf16 (exact).  MW = 32:
// v_mfma_scale_f32_32x32x64_f8f6f4 (native) or v_mfma_f32_32x32x16_bf16
// (exact); every 16-byte LDS read then feeds whole instructions.
// Accumulator element v of a lane holds
//   MW = 16: row 4 * (lane / 16) + v,                         column lane % 16
//   MW = 32: row 8 * (v / 4) + 4 * (lane / 32) + v % 4,      column lane % 32
// of its 16 x 16 (32 x 32) output block.
typedef float v16f __attribute__((ext_vector_type(16)));

template <int MW>
struct AccT;
template <>
struct AccT<16> { typedef v4f T; static constexpr int N = 4; };
template <>
struct AccT<32> { typedef v16f T; static constexpr int N = 16; };

template <int BM, int BN, int WGM, int WGN, int OCC, bool EXACT, int MW>
__global__ void __launch_bounds__(WGM * WGN * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
mxgemm_kernel(GemmArgs p)
{
    constexpr int NW = WGM * WGN;
    constexpr int NT = NW * 64;
    constexpr int TM = BM / WGM, TN = BN / WGN;
    constexpr int GA = TM / MW, GB = TN / MW;
    static_assert(TM % MW == 0 && TN % MW == 0, "wave tile must be a multiple of the MFMA width");
    static_assert(BM % 8 == 0 && BN % 8 == 0, "tile rows come in groups of 8");
    typedef typename AccT<MW>::T acc_t;
    constexpr int NACC = AccT<MW>::N;
    constexpr int A_BYTES = BM * kBK, B_BYTES = BN * kBK;
    // scale bytes: 4 per row and K-step; padded to one 64-lane copy
    constexpr int SA_BYTES = 4 * (BM > 64 ? BM : 64), SB_BYTES = 4 * (BN > 64 ? BN : 64);
    constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
    constexpr int IA = BM / 8, IB = BN / 8;            // 1 KB copies per K-step
    constexpr int JA = (IA + NW - 1) / NW, JB = (IB + NW - 1) / NW;
    constexpr int ISA = (BM + 63) / 64, ISB = (BN + 63) / 64;   // scale copies

    // Two distinct LDS objects (not one array indexed by the step parity):
    // the compiler then knows a step's copies into one stage never alias
    // the reads of the other, and does not wait for the copies before the
    // reads.
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[STAGE];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int lr = lane & (MW - 1);         // row / column of the lane in a block
    const int lq = lane / MW;               // lane group

    const int steps_per_seg = p.kpr / kBK;
    const int sk = p.kpr >> 5;              // scale bytes per row per segment
    const int K32 = p.K >> 5;

    for (int w = remap_block(blockIdx.x, gridDim.x); w < p.total_work; w += gridDim.x) {
        const TileCoord tc = decode_work(w, p.tiles_m, p.tiles_n, p.split, p.group_n);
        const int m0 = tc.tm * BM, n0 = tc.tn * BN;

        // Per-lane 32-bit source offsets of this wave's copies.  A offsets
        // are relative to the window's ring base (the ring is < 2 GiB), B
        // offsets relative to row n0 of B.  Rows past the edge are clamped
        // to the last valid row; their results are never stored.
        uint32_t a_off[JA], b_off[JB], as_off[ISA], bs_off[ISB];
#pragma unroll
        for (int j = 0; j < JA; ++j) {
            const int t = wave + j * NW;                 // copy index
            const int row = 8 * (t < IA ? t : IA - 1) + (lane >> 3);
            const int ch = swz_t<MW>(row, lane & 7);
            int g = m0 + row;
            g = g < p.rows ? g : p.rows - 1;
            a_off[j] = (uint32_t)((g / p.cms) * p.a_slot_stride) + (uint32_t)((g % p.cms) * p.kpr) + ch * 16;
        }
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            const int t = wave + j * NW;
            const int row = 8 * (t < IB ? t : IB - 1) + (lane >> 3);
            const int ch = swz_t<MW>(row, lane & 7);
            int g = n0 + row < p.N ? row : p.N - 1 - n0;
            b_off[j] = (uint32_t)g * (uint32_t)p.K + ch * 16;
        }
#pragma unroll
        for (int j = 0; j < ISA; ++j) {
            int row = 64 * j + lane;
            row = row < BM ? row : BM - 1;
            int g = m0 + row;
            g = g < p.rows ? g : p.rows - 1;
            as_off[j] = (uint32_t)((g / p.cms) * p.as_slot_stride) + (uint32_t)((g % p.cms) * sk);
        }
#pragma unroll
        for (int j = 0; j < ISB; ++j) {
            int row = 64 * j + lane;
            row = row < BN ? row : BN - 1;
            int g = n0 + row < p.N ? row : p.N - 1 - n0;
            bs_off[j] = (uint32_t)g * (uint32_t)K32;
        }
        const uint8_t* __restrict__ bt = p.b + (int64_t)n0 * p.K;
        const uint8_t* __restrict__ bst = p.bs + (int64_t)n0 * K32;

        const int seg0 = tc.ks * p.segs_per_split;
        const int nsteps = p.segs_per_split * steps_per_seg;

        acc_t acc[GA][GB];
#pragma unroll
        for (int i = 0; i < GA; ++i)
#pragma unroll
            for (int j = 0; j < GB; ++j)
#pragma unroll
                for (int v = 0; v < NACC; ++v)
                    acc[i][j][v] = 0.f;

// issue the copies of K-step S into stage DST
#define MXG_COPY_STEP(S, DST)                                                              \
    do {                                                                                   \
        const int seg_ = seg0 + (S) / steps_per_seg;                                       \
        const int kk_ = ((S) % steps_per_seg) * kBK;                                       \
        const uint8_t* a_ = p.a + (int64_t)seg_ * p.cms * p.kpr + kk_;                      \
        const uint8_t* b_ = bt + (int64_t)seg_ * p.kpr + kk_;                               \
        const uint8_t* as_ = p.as + (int64_t)seg_ * p.cms * sk + (kk_ >> 5);                \
        const uint8_t* bs_ = bst + (((int64_t)seg_ * p.kpr + kk_) >> 5);                    \
        uint8_t* st_ = (DST);                                                              \
        _Pragma("unroll") for (int j = 0; j < JA; ++j)                                     \
            if (IA % NW == 0 || wave + j * NW < IA)                                        \
                dma16(a_ + a_off[j], st_ + (wave + j * NW) * 1024);                        \
        _Pragma("unroll") for (int j = 0; j < JB; ++j)                                     \
            if (IB % NW == 0 || wave + j * NW < IB)                                        \
                dma16(b_ + b_off[j], st_ + A_BYTES + (wave + j * NW) * 1024);              \
        if (wave == 0) {                                                                   \
            _Pragma("unroll") for (int j = 0; j < ISA; ++j)                                \
                dma4(as_ + as_off[j], st_ + A_BYTES + B_BYTES + j * 256);                  \
        }                                                                                  \
        if (wave == NW - 1) {                                                              \
            _Pragma("unroll") for (int j = 0; j < ISB; ++j)                                \
                dma4(bs_ + bs_off[j], st_ + A_BYTES + B_BYTES + SA_BYTES + j * 256);       \
        }                                                                                  \
    } while (0)

        __syncthreads();   // the previous work item is done with the LDS
        MXG_COPY_STEP(0, stage0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();

        // One K-step: start the copy of step s + 1 into NXT, multiply the
        // tiles in CUR, then wait for the copy and synchronise.
        auto kstep = [&](int s, const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt) {
            if (s + 1 < nsteps)
                MXG_COPY_STEP(s + 1, nxt);

            const uint8_t* sa_ = cur;
            const uint8_t* sb_ = sa_ + A_BYTES;
            const uint8_t* ssa = sb_ + B_BYTES;
            const uint8_t* ssb = ssa + SA_BYTES;
            // Row r of a fragment group is r = group base + lr with the
            // group base a multiple of MW >= 16, so r & 7 = lr & 7: a lane's
            // swizzled byte offsets differ between groups by a constant.
            const uint8_t* pa = sa_ + (wm * TM + lr) * kBK;
            const uint8_t* pb = sb_ + (wn * TN + lr) * kBK;
            const uint8_t* psa = ssa + (wm * TM + lr) * 4;
            const uint8_t* psb = ssb + (wn * TN + lr) * 4;
            auto chunk = [&](int c) { return swz_t<MW>(lr, c) * 16; };

            if constexpr (!EXACT && MW == 16) {
                // Native, 16 x 16 x 128: one scaled MFMA per (A group, B
                // group) per K-step.  Lane group q holds K [16q, 16q + 16)
                // and [64 + 16q, ...); its scale byte is MX block q.  A
                // fragments double buffered so group i + 1 is in flight
                // while group i's MFMAs run.
                const int off_lo = chunk(lq), off_hi = chunk(lq + 4);
                v8i bf[GB];
                int sbv[GB];
#pragma unroll
                for (int j = 0; j < GB; ++j) {
                    const u32x4 lo = *reinterpret_cast<const u32x4*>(pb + j * MW * kBK + off_lo);
                    const u32x4 hi = *reinterpret_cast<const u32x4*>(pb + j * MW * kBK + off_hi);
                    bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    sbv[j] = psb[j * MW * 4 + lq];
                }
                v8i af[2];
                int sav[2];
                {
                    const u32x4 lo = *reinterpret_cast<const u32x4*>(pa + off_lo);
                    const u32x4 hi = *reinterpret_cast<const u32x4*>(pa + off_hi);
                    af[0] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    sav[0] = psa[lq];
                }
#pragma unroll
                for (int i = 0; i < GA; ++i) {
                    const int cur = i & 1;
                    if (i + 1 < GA) {
                        const u32x4 lo = *reinterpret_cast<const u32x4*>(pa + (i + 1) * MW * kBK + off_lo);
                        const u32x4 hi = *reinterpret_cast<const u32x4*>(pa + (i + 1) * MW * kBK + off_hi);
                        af[cur ^ 1] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                          (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                        sav[cur ^ 1] = psa[(i + 1) * MW * 4 + lq];
                    }
#pragma unroll
                    for (int j = 0; j < GB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            af[cur], bf[j], acc[i][j], 0 /*A: E4M3*/, 0 /*B: E4M3*/,
                            0, sav[cur], 0, sbv[j]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else if constexpr (!EXACT && MW == 32) {
                // Native, 32 x 32 x 64: two scaled MFMAs (m = 0, 1: K
                // [64m, 64m + 64)) per (A group, B group) per K-step.  Lane
                // group h = lane / 32 holds K [64m + 16h, +16) and
                // [64m + 32 + 16h, +16); its scale byte is MX block 2m + h.
                v8i bf[GB][2];
                int sbv[GB][2];
#pragma unroll
                for (int j = 0; j < GB; ++j)
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        const u32x4 lo = *reinterpret_cast<const u32x4*>(pb + j * MW * kBK + chunk(4 * m + lq));
                        const u32x4 hi = *reinterpret_cast<const u32x4*>(pb + j * MW * kBK + chunk(4 * m + 2 + lq));
                        bf[j][m] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                        sbv[j][m] = psb[j * MW * 4 + 2 * m + lq];
                    }
                v8i af[2][2];
                int sav[2][2];
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const u32x4 lo = *reinterpret_cast<const u32x4*>(pa + chunk(4 * m + lq));
                    const u32x4 hi = *reinterpret_cast<const u32x4*>(pa + chunk(4 * m + 2 + lq));
                    af[0][m] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    sav[0][m] = psa[2 * m + lq];
                }
#pragma unroll
                for (int i = 0; i < GA; ++i) {
                    const int cur = i & 1;
                    if (i + 1 < GA) {
#pragma unroll
                        for (int m = 0; m < 2; ++m) {
                            const u32x4 lo = *reinterpret_cast<const u32x4*>(pa + (i + 1) * MW * kBK + chunk(4 * m + lq));
                            const u32x4 hi = *reinterpret_cast<const u32x4*>(pa + (i + 1) * MW * kBK + chunk(4 * m + 2 + lq));
                            af[cur ^ 1][m] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                            sav[cur ^ 1][m] = psa[(i + 1) * MW * 4 + 2 * m + lq];
                        }
                    }
                    // m outer: consecutive MFMAs update different
                    // accumulators, so none waits for the one before
#pragma unroll
                    for (int m = 0; m < 2; ++m)
#pragma unroll
                        for (int j = 0; j < GB; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                af[cur][m], bf[j][m], acc[i][j], 0 /*A: E4M3*/, 0 /*B: E4M3*/,
                                0, sav[cur][m], 0, sbv[j][m]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else if constexpr (EXACT && MW == 16) {
                // Exact, 16 x 16 x 32 bf16: each MX block j is one MFMA.
                // Lane group q takes 8 codes of block j (K [32j + 8q, +8)),
                // converted to bfloat16 with the block's scale folded in
                // (exact: 4-bit significands times a power of two).  A and
                // B use the same K assignment, so every product pairs
                // correctly; products are exact in the MFMA and summed with
                // FP32-grade precision.
                uint32_t sa_w[GA], sb_w[GB];
#pragma unroll
                for (int g = 0; g < GB; ++g)
                    sb_w[g] = *reinterpret_cast<const uint32_t*>(psb + g * MW * 4);
#pragma unroll
                for (int i = 0; i < GA; ++i)
                    sa_w[i] = *reinterpret_cast<const uint32_t*>(psa + i * MW * 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int lane_off = chunk(2 * j + (lq >> 1)) + (lq & 1) * 8;
                    u32x2 rb[GB], ra[GA];
#pragma unroll
                    for (int g = 0; g < GB; ++g)
                        rb[g] = *reinterpret_cast<const u32x2*>(pb + g * MW * kBK + lane_off);
#pragma unroll
                    for (int i = 0; i < GA; ++i)
                        ra[i] = *reinterpret_cast<const u32x2*>(pa + i * MW * kBK + lane_off);
                    v8bf bb[GB];
#pragma unroll
                    for (int g = 0; g < GB; ++g)
                        bb[g] = fp8x8_to_bf16(rb[g], e8m0_to_f32(sb_w[g] >> (8 * j)));
                    v8bf ab[2];
                    ab[0] = fp8x8_to_bf16(ra[0], e8m0_to_f32(sa_w[0] >> (8 * j)));
#pragma unroll
                    for (int i = 0; i < GA; ++i) {
                        const int cur = i & 1;
#pragma unroll
                        for (int g = 0; g < GB; ++g)
                            acc[i][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab[cur], bb[g], acc[i][g], 0, 0, 0);
                        if (i + 1 < GA)
                            ab[cur ^ 1] = fp8x8_to_bf16(ra[i + 1], e8m0_to_f32(sa_w[i + 1] >> (8 * j)));
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            } else {
                // Exact, 32 x 32 x 16 bf16: MX block j is two MFMAs
                // (m = 0, 1).  Lane group h = lane / 32 takes K
                // [32j + 16h + 8m, +8) in MFMA m, so one 16-byte read of
                // logical chunk 2j + h feeds both.  Codes are converted to
                // bfloat16 with the block scale folded in (exact), A and B
                // share the K assignment.
                uint32_t sa_w[GA], sb_w[GB];
#pragma unroll
                for (int g = 0; g < GB; ++g)
                    sb_w[g] = *reinterpret_cast<const uint32_t*>(psb + g * MW * 4);
#pragma unroll
                for (int i = 0; i < GA; ++i)
                    sa_w[i] = *reinterpret_cast<const uint32_t*>(psa + i * MW * 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int off = chunk(2 * j + lq);
                    u32x4 rb[GB], ra[GA];
#pragma unroll
                    for (int g = 0; g < GB; ++g)
                        rb[g] = *reinterpret_cast<const u32x4*>(pb + g * MW * kBK + off);
#pragma unroll
                    for (int i = 0; i < GA; ++i)
                        ra[i] = *reinterpret_cast<const u32x4*>(pa + i * MW * kBK + off);
                    v8bf bb[GB][2];
#pragma unroll
                    for (int g = 0; g < GB; ++g) {
                        const float sc = e8m0_to_f32(sb_w[g] >> (8 * j));
                        bb[g][0] = fp8x8_to_bf16(u32x2{rb[g].x, rb[g].y}, sc);
                        bb[g][1] = fp8x8_to_bf16(u32x2{rb[g].z, rb[g].w}, sc);
                    }
                    v8bf ab[2][2];
                    {
                        const float sc = e8m0_to_f32(sa_w[0] >> (8 * j));
                        ab[0][0] = fp8x8_to_bf16(u32x2{ra[0].x, ra[0].y}, sc);
                        ab[0][1] = fp8x8_to_bf16(u32x2{ra[0].z, ra[0].w}, sc);
                    }
#pragma unroll
                    for (int i = 0; i < GA; ++i) {
                        const int cur = i & 1;
#pragma unroll
                        for (int m = 0; m < 2; ++m)
#pragma unroll
                            for (int g = 0; g < GB; ++g)
                                acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab[cur][m], bb[g][m], acc[i][g], 0, 0, 0);
                        if (i + 1 < GA) {
                            const float sc = e8m0_to_f32(sa_w[i + 1] >> (8 * j));
                            ab[cur ^ 1][0] = fp8x8_to_bf16(u32x2{ra[i + 1].x, ra[i + 1].y}, sc);
                            ab[cur ^ 1][1] = fp8x8_to_bf16(u32x2{ra[i + 1].z, ra[i + 1].w}, sc);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }

            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        };
        for (int s = 0; s < nsteps; s += 2) {
            kstep(s, stage0, stage1);
            if (s + 1 < nsteps)
                kstep(s + 1, stage1, stage0);
        }
#undef MXG_COPY_STEP

        // ---- epilogue --------------------------------------------------
        // (row, column) in C of accumulator element v of block (i, j)
        auto out_row = [&](int i, int v) {
            return MW == 16 ? m0 + wm * TM + i * 16 + 4 * lq + v
                            : m0 + wm * TM + i * 32 + 8 * (v >> 2) + 4 * lq + (v & 3);
        };
        auto out_col = [&](int j) { return n0 + wn * TN + j * MW + lr; };
        if (p.split == 1) {
#pragma unroll
            for (int i = 0; i < GA; ++i)
#pragma unroll
                for (int j = 0; j < GB; ++j) {
                    const int col = out_col(j);
#pragma unroll
                    for (int v = 0; v < NACC; ++v) {
                        const int row = out_row(i, v);
                        if (row < p.rows && col < p.N)
                            p.c[(int64_t)row * p.N + col] = f32_to_bf16_rne(acc[i][j][v]);
                    }
                }
        } else {
            // Split-K: every split stores its FP32 partial tile; the last
            // split to arrive sums all partials in split order (so the
            // result does not depend on arrival order) and writes C.
            constexpr int NQ = NACC / 4;
            const int tile_id = tc.tm * p.tiles_n + tc.tn;
            float* wsp = p.ws + ((int64_t)tile_id * p.split + tc.ks) * (BM * BN);
#pragma unroll
            for (int i = 0; i < GA; ++i)
#pragma unroll
                for (int j = 0; j < GB; ++j)
#pragma unroll
                    for (int q = 0; q < NQ; ++q)
                        *reinterpret_cast<v4f*>(wsp + (((i * GB + j) * NQ + q) * NT + tid) * 4) =
                            v4f{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                acc[i][j][4 * q + 3]};
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
                        const int col = out_col(j);
#pragma unroll
                        for (int q = 0; q < NQ; ++q) {
                            const int64_t off = (((i * GB + j) * NQ + q) * NT + tid) * 4;
                            v4f sum = *reinterpret_cast<const v4f*>(wst + off);
                            for (int s = 1; s < p.split; ++s) {
                                const v4f t = *reinterpret_cast<const v4f*>(wst + (int64_t)s * (BM * BN) + off);
                                sum[0] += t[0];
                                sum[1] += t[1];
                                sum[2] += t[2];
                                sum[3] += t[3];
                            }
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                const int row = out_row(i, 4 * q + u);
                                if (row < p.rows && col < p.N)
                                    p.c[(int64_t)row * p.N + col] = f32_to_bf16_rne(sum[u]);
                            }
                        }
                    }
                if (tid == 0)
                    atomicExch(p.counters + tile_id, 0);
            }
        }
    }
}

template <int BM, int BN, int WGM, int WGN, int OCC, int MW>
static hipError_t launch_cfg(const GemmArgs& a, int grid, bool exact, hipStream_t stream)
{
    if (exact)
        hipLaunchKernelGGL((mxgemm_kernel<BM, BN, WGM, WGN, OCC, true, MW>), dim3(grid),
                           dim3(WGM * WGN * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((mxgemm_kernel<BM, BN, WGM, WGN, OCC, false, MW>), dim3(grid),
                           dim3(WGM * WGN * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_gemm(int cfg, bool exact, const GemmArgs& a, int grid, hipStream_t stream)
{
    switch (cfg) {
    case 0: return launch_cfg<256, 256, 2, 4, 2, 32>(a, grid, exact, stream);
    case 1: return launch_cfg<256, 128, 2, 2, 1, 32>(a, grid, exact, stream);
    case 2: return launch_cfg<128, 128, 2, 2, 1, 32>(a, grid, exact, stream);
    case 3: return launch_cfg<64, 64, 2, 2, 4, 16>(a, grid, exact, stream);
    case 4: return launch_cfg<32, 64, 1, 4, 4, 16>(a, grid, exact, stream);
    case 5: return launch_cfg<16, 64, 1, 4, 4, 16>(a, grid, exact, stream);
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
