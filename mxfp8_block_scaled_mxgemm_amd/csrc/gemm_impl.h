// The block-scaled GEMM kernels, templated on the FP8 formats of A and B.
// Each format pair is instantiated in its own translation unit.
#pragma once

#include <type_traits>

#include "device_util.h"
#include "schedule.h"

namespace mxg {

// Block-scaled GEMM over one window of staged rows.
//
// Work-group tile BM x BN, K-step 128 (four MX blocks).  Each K-step's A and
// B tiles and their scale bytes are copied global -> LDS by the load unit
// itself (global_load_lds), double-buffered, so the next step's copy runs
// while the current one is multiplied and no registers hold staged data.
// A lane of a copy instruction writes 16 bytes at lds_base + 16 * lane:
// eight lanes fill one 128-byte tile row, and lane L fetches the logical
// chunk that the row's XOR swizzle places at physical chunk L % 8.
//
// MFMA forms and accumulator layouts (MW = MFMA width):
//   MW = 16: v_mfma_scale_f32_16x16x128_f8f6f4 (native) or
//            v_mfma_f32_16x16x32_bf16 (exact); element v of a lane holds
//            row 4 * (lane / 16) + v, column lane % 16;
//   MW = 32: v_mfma_scale_f32_32x32x64_f8f6f4 (native) or
//            v_mfma_f32_32x32x16_bf16 (exact); element v holds row
//            8 * (v / 4) + 4 * (lane / 32) + v % 4, column lane % 32
// of its MW x MW output block.
// LDS stage layout of a BM x BN tile pair: A rows, B rows (128 bytes each),
// then 4 scale bytes per A row and per B row (padded to one 64-lane copy).
template <int BM, int BN, int NW>
struct StageGeom {
    static constexpr int A_BYTES = BM * kBK, B_BYTES = BN * kBK;
    static constexpr int SA_BYTES = 4 * (BM > 64 ? BM : 64), SB_BYTES = 4 * (BN > 64 ? BN : 64);
    static constexpr int SA_OFF = A_BYTES + B_BYTES, SB_OFF = SA_OFF + SA_BYTES;
    static constexpr int STAGE = SB_OFF + SB_BYTES;
    static constexpr int IA = BM / 8, IB = BN / 8;                  // 1 KB copies per K-step
    static constexpr int JA = (IA + NW - 1) / NW, JB = (IB + NW - 1) / NW;
    static constexpr int ISA = (BM + 63) / 64, ISB = (BN + 63) / 64; // 256-byte scale copies
    static constexpr int KSA = (ISA + NW - 1) / NW, KSB = (ISB + NW - 1) / NW;
};

// The copies of one work item: per-lane 32-bit source offsets, fixed for
// the item.  A offsets are relative to the window's ring base (the ring is
// < 2 GiB), B offsets relative to row n0 of B.  Rows past the edge are
// clamped to the last valid row; their results are never stored.
template <int BM, int BN, int NW, int MW>
struct CopyOffsets {
    typedef StageGeom<BM, BN, NW> G;
    uint32_t a[G::JA], b[G::JB], as[G::KSA], bs[G::KSB];
};

template <int BM, int BN, int NW, int MW>
__device__ __forceinline__ void copy_offsets(const GemmArgs& p, int m0, int n0, int wave, int lane,
                                             CopyOffsets<BM, BN, NW, MW>& o)
{
    typedef StageGeom<BM, BN, NW> G;
    const int sk = p.kpr >> 5;
    const int K32 = p.K >> 5;
#pragma unroll
    for (int j = 0; j < G::JA; ++j) {
        const int t = wave + j * NW;
        const int row = 8 * (t < G::IA ? t : G::IA - 1) + (lane >> 3);
        const int ch = swz_t<MW>(row, lane & 7);
        int g = m0 + row;
        g = g < p.rows ? g : p.rows - 1;
        o.a[j] = (uint32_t)((g / p.cms) * p.a_slot_stride) + (uint32_t)((g % p.cms) * p.kpr) + ch * 16;
    }
#pragma unroll
    for (int j = 0; j < G::JB; ++j) {
        const int t = wave + j * NW;
        const int row = 8 * (t < G::IB ? t : G::IB - 1) + (lane >> 3);
        const int ch = swz_t<MW>(row, lane & 7);
        const int g = n0 + row < p.N ? row : p.N - 1 - n0;
        o.b[j] = (uint32_t)g * (uint32_t)p.K + ch * 16;
    }
#pragma unroll
    for (int j = 0; j < G::KSA; ++j) {
        const int t = wave + j * NW;
        int row = 64 * (t < G::ISA ? t : G::ISA - 1) + lane;
        row = row < BM ? row : BM - 1;
        int g = m0 + row;
        g = g < p.rows ? g : p.rows - 1;
        o.as[j] = (uint32_t)((g / p.cms) * p.as_slot_stride) + (uint32_t)((g % p.cms) * sk);
    }
#pragma unroll
    for (int j = 0; j < G::KSB; ++j) {
        const int t = wave + j * NW;
        int row = 64 * (t < G::ISB ? t : G::ISB - 1) + lane;
        row = row < BN ? row : BN - 1;
        const int g = n0 + row < p.N ? row : p.N - 1 - n0;
        o.bs[j] = (uint32_t)g * (uint32_t)K32;
    }
}

// Global addresses of K-step s of a work item whose first segment is seg0
// and whose B tile starts at row n0 (all wave-uniform).
struct StepSrc {
    const uint8_t* a;
    const uint8_t* b;
    const uint8_t* as;
    const uint8_t* bs;
};

__device__ __forceinline__ StepSrc step_src(const GemmArgs& p, int seg0, int n0, int s)
{
    const int steps_per_seg = p.kpr / kBK;
    const int sk = p.kpr >> 5;
    const int seg = seg0 + s / steps_per_seg;
    const int kk = (s % steps_per_seg) * kBK;
    StepSrc r;
    r.a = p.a + (int64_t)seg * p.cms * p.kpr + kk;
    r.b = p.b + (int64_t)n0 * p.K + (int64_t)seg * p.kpr + kk;
    r.as = p.as + (int64_t)seg * p.cms * sk + (kk >> 5);
    r.bs = p.bs + (((int64_t)n0 * p.K + (int64_t)seg * p.kpr + kk) >> 5);
    return r;
}

// Issue the copies of one K-step (sources `src`) into the stage at dst.
// With nparts > 1 only share `part` of them (copies j with
// j % nparts == part), so the issue can be spread between other work.
template <int BM, int BN, int NW, int MW>
__device__ __forceinline__ void copy_issue(const CopyOffsets<BM, BN, NW, MW>& o, const StepSrc& src, uint8_t* dst,
                                           int wave, int part = 0, int nparts = 1, uint8_t* pad = nullptr)
{
    typedef StageGeom<BM, BN, NW> G;
    // With `pad`, a wave with no piece left in a slot copies 4 bytes per
    // lane into the 256 bytes at `pad` instead, so every wave issues the
    // same number of copy instructions (and can count them with vmcnt).
#pragma unroll
    for (int j = 0; j < G::JA; ++j)
        if (j % nparts == part) {
            if (G::IA % NW == 0 || wave + j * NW < G::IA)
                dma16_at(src.a, o.a[j], dst + (wave + j * NW) * 1024);
            else if (pad)
                dma4_at(src.as, o.as[0], pad);
        }
#pragma unroll
    for (int j = 0; j < G::JB; ++j)
        if (j % nparts == part) {
            if (G::IB % NW == 0 || wave + j * NW < G::IB)
                dma16_at(src.b, o.b[j], dst + G::A_BYTES + (wave + j * NW) * 1024);
            else if (pad)
                dma4_at(src.as, o.as[0], pad);
        }
#pragma unroll
    for (int j = 0; j < G::KSA; ++j)
        if (j % nparts == part) {
            if (G::ISA % NW == 0 || wave + j * NW < G::ISA)
                dma4_at(src.as, o.as[j], dst + G::SA_OFF + (wave + j * NW) * 256);
            else if (pad)
                dma4_at(src.as, o.as[0], pad);
        }
#pragma unroll
    for (int j = 0; j < G::KSB; ++j)
        if ((j + 1) % nparts == part) {
            if (G::ISB % NW == 0 || wave + j * NW < G::ISB)
                dma4_at(src.bs, o.bs[j], dst + G::SB_OFF + (wave + j * NW) * 256);
            else if (pad)
                dma4_at(src.as, o.as[0], pad);
        }
}

// Wait until at most n of this wave's copy instructions are outstanding
// (n a compile-time count; vmcnt holds 0..63 on gfx950).
template <int N>
__device__ __forceinline__ void wait_copies()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait_copies<r * CPW>() for the runtime r = rem in [0, R]
template <int CPW, int R>
__device__ __forceinline__ void wait_steps(int rem)
{
    if constexpr (R >= 0) {
        if (rem == R) {
            wait_copies<R * CPW>();
            return;
        }
        wait_steps<CPW, R - 1>(rem);
    }
}

// Write a wave's accumulators: GA x GB blocks of MW x MW, block (i, j)
// covering rows row0 + MW i and columns col0 + MW j of C.  Every MFMA takes
// the B fragment as its first operand (it computes the transposed block),
// so element v of a lane holds row lane % MW and column
//   MW = 32: 8 (v / 4) + 4 (lane / 32) + v % 4,
//   MW = 16: 4 (lane / 16) + v:
// four consecutive columns per v / 4, written as one 8-byte (C) or 16-byte
// (split-K partial) store where the layout allows.  With split > 1 the
// FP32 partial goes to ws[split index][row][column] and a second kernel
// sums the splits.
template <int GA, int GB, int MW, typename acc_t>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const TileCoord& tc, acc_t (&acc)[GA][GB],
                                           int row0, int col0, int lane)
{
    constexpr int NQ = AccT<MW>::N / 4;
    const int lr = lane & (MW - 1), lq = lane / MW;
    // The lane's first element.  Hidden from the optimiser: otherwise the
    // lane-dependent parts of every store address are computed up front
    // and held in registers across the K loop.
    int64_t lane_base = (int64_t)(row0 + lr) * p.N + col0 + 4 * lq;
    asm volatile("" : "+v"(lane_base));
    const bool partial = p.split > 1;
    const bool vec = partial ? (p.N & 3) == 0 : p.c_vec4 != 0;
    float* wsp = p.ws + (int64_t)tc.ks * p.rows * p.N;
#pragma unroll
    for (int i = 0; i < GA; ++i) {
        if (row0 + i * MW + lr >= p.rows)
            continue;
#pragma unroll
        for (int j = 0; j < GB; ++j)
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int cofs = j * MW + (MW == 32 ? 8 * q : 0);
                const int col = col0 + 4 * lq + cofs;
                const int64_t off = lane_base + (int64_t)(i * MW) * p.N + cofs;
                const v4f x = v4f{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                if (vec && col + 3 < p.N) {
                    if (partial && p.fused)
                        st_dev16(wsp + off, __builtin_bit_cast(u32x4, x));
                    else if (partial)
                        *reinterpret_cast<v4f*>(wsp + off) = x;
                    else
                        *reinterpret_cast<u32x2*>(p.c + off) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (col + u < p.N) {
                            if (partial && p.fused)
                                st_dev(wsp + off + u, x[u]);
                            else if (partial)
                                wsp[off + u] = x[u];
                            else
                                p.c[off + u] = f32_to_bf16_rne(x[u]);
                        }
                }
            }
    }
}

// Write a wave's TM x TN accumulators (32 x 32 MFMA blocks, layout as in
// store_tile) as bfloat16 to C through the wave's own LDS region `buf`
// (TM * TN * 2 bytes), so that the global stores are whole rows: a store
// instruction writes 64 / (TN / 8) rows of TN * 2 contiguous bytes instead
// of 32 rows of 16 bytes.  In `buf` row r holds its TN / 8 16-byte chunks
// XOR-swizzled by r, so neither the 8-byte writes (32 rows, one column
// chunk) nor the 16-byte reads (whole rows) pile onto a few banks.  Needs C
// 16-byte aligned with N % 8 == 0; rows and column chunks past the edge are
// not stored.
template <int GA, int GB, int TM, int TN>
__device__ __forceinline__ void store_tile_lds(const GemmArgs& p, v16f (&acc)[GA][GB], uint8_t* buf,
                                               int row0, int col0, int lane)
{
    constexpr int RB = TN * 2;           // bytes per row in buf
    constexpr int CPR = TN / 8;          // 16-byte chunks per row
    static_assert(GA * 32 == TM && GB * 32 == TN && (CPR & (CPR - 1)) == 0 && CPR <= 64,
                  "wave tile of whole 32 x 32 blocks, a power-of-two number of row chunks");
    const int lr = lane & 31, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < GA; ++i)
#pragma unroll
        for (int j = 0; j < GB; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // columns 32 j + 8 q + 4 h + (0..3): chunk 4 j + q, bytes 8 h..8 h + 7
                const int r = 32 * i + lr;
                const int c = 4 * j + q;
                *reinterpret_cast<u32x2*>(buf + r * RB + ((c ^ (r & (CPR - 1))) * 16) + 8 * h) =
                    u32x2{pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                          pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
            }
    // LDS operations of one wave complete in order; the wave reads back only
    // what it wrote itself
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    constexpr int RPI = 64 / CPR;        // rows per store instruction
    const int cl = lane % CPR, rl = lane / CPR;
#pragma unroll
    for (int t = 0; t < TM / RPI; ++t) {
        const int r = t * RPI + rl;
        const u32x4 v = *reinterpret_cast<const u32x4*>(buf + r * RB + ((cl ^ (r & (CPR - 1))) * 16));
        const int grow = row0 + r, gcol = col0 + 8 * cl;
        if (grow < p.rows && gcol < p.N)
            *reinterpret_cast<u32x4*>(p.c + (int64_t)grow * p.N + gcol) = v;
    }
}

// K groups (WGK groups of NWG waves sharing one tile, each summing its own
// share of the K-steps into v16f accumulators of GA x GB 32 x 32 blocks):
// groups 1 .. WGK - 1 leave their sums in `red` (elements 4q .. 4q + 3 of
// block b of a lane as one 16-byte piece at float (b * 4 + q) * 256 + 4 *
// lane of the wave's slot of GA * GB * 1024 floats), and group 0 adds them
// in group order.  Every thread of the work-group calls it: the first
// barrier ends the K loop's LDS reads, the second publishes the sums.
template <int NWG, int WGK, int GA, int GB>
__device__ __forceinline__ void reduce_k_groups(v16f (&acc)[GA][GB], float* red, int wk, int wl, int lane)
{
    constexpr int SLOT = GA * GB * 1024;
    __syncthreads();
    if (wk > 0) {
        float* slot = red + ((wk - 1) * NWG + wl) * SLOT;
#pragma unroll
        for (int i = 0; i < GA; ++i)
#pragma unroll
            for (int g = 0; g < GB; ++g)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<v4f*>(slot + ((i * GB + g) * 4 + q) * 256 + 4 * lane) =
                        v4f{acc[i][g][4 * q], acc[i][g][4 * q + 1], acc[i][g][4 * q + 2], acc[i][g][4 * q + 3]};
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll 1
        for (int k = 1; k < WGK; ++k) {
            const float* slot = red + ((k - 1) * NWG + wl) * SLOT;
#pragma unroll
            for (int i = 0; i < GA; ++i)
#pragma unroll
                for (int g = 0; g < GB; ++g)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const v4f x = *reinterpret_cast<const v4f*>(slot + ((i * GB + g) * 4 + q) * 256 + 4 * lane);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[i][g][4 * q + e] += x[e];
                    }
        }
    }
}

// Split-K, fused combine: once this work-group's partials are stored
// (device-scope), count its arrival at the tile; the last split to arrive
// sums the tile's partials in split order into C and sets the count back to
// zero for the next launch.  Nothing waits, so the grid need not be
// resident at once.
template <int BM, int BN>
__device__ __forceinline__ void split_combine(const GemmArgs& p, const TileCoord& tc, int m0, int n0)
{
    __shared__ uint32_t s_last;
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t* cnt = p.tile_cnt + tc.tm * p.tiles_n + tc.tn;
        const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = old == (uint32_t)(p.split - 1);
        if (s_last)
            __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last)
        return;
    const int nr = p.rows - m0 < BM ? p.rows - m0 : BM;
    combine_tile(p.ws, (int64_t)p.rows * p.N, p.c, m0, nr, n0, BN, p.N, p.split, p.c_vec4 != 0);
}

// Block-scaled GEMM, scaled-MFMA (native) forms and the 16-wide exact form.
// WGM x WGN waves of (BM / WGM) x (BN / WGN).  A stage holds CH K-steps, so
// small tiles keep several K-steps' copies in flight (their K loop is bound
// by copy latency, not by the MFMAs).  ONE: a work item has at most CH
// K-steps, all copied at once into a single stage (skinny shapes, where the
// whole K range of a split fits in LDS).  WGK > 1 (native 32-wide form
// only): K groups as in mxgemm_exact_kernel -- WGK groups of WGM x WGN waves
// share the tile, group k taking K-steps k, k + WGK, ...; a stage holds one
// K-step per group, copied by that group; the groups' sums are added in
// group order at the end.
template <int BM, int BN, int WGM, int WGN, int OCC, bool EXACT, int MW, int CH, bool ONE, int FA, int FB,
          int WGK = 1>
__global__ void __launch_bounds__(WGM * WGN * WGK * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
mxgemm_kernel(GemmArgs p)
{
    static_assert(WGK == 1 || (!EXACT && MW == 32 && CH == 1 && !ONE), "K groups: native 32-wide form, CH = 1");
    constexpr int NWG = WGM * WGN;          // waves of one K group
    constexpr int NW = NWG * WGK;
    constexpr int TM = BM / WGM, TN = BN / WGN;
    constexpr int GA = TM / MW, GB = TN / MW;
    static_assert(TM % MW == 0 && TN % MW == 0, "wave tile must be a multiple of the MFMA width");
    static_assert(BM % 8 == 0 && BN % 8 == 0, "tile rows come in groups of 8");
    static_assert(!(EXACT && MW == 32), "the 32-wide exact form is mxgemm_exact_kernel");
    typedef typename AccT<MW>::T acc_t;
    constexpr int NACC = AccT<MW>::N;
    typedef StageGeom<BM, BN, NWG> G;       // one K-step, copied by one K group

    // Two distinct LDS objects (not one array indexed by the step parity):
    // the compiler then knows a step's copies into one stage never alias
    // the reads of the other, and does not wait for the copies before the
    // reads.  Sub-stage c * WGK + k holds K-step c of the stage for group k.
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[CH * WGK * G::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[ONE ? 16 : CH * WGK * G::STAGE];
    __shared__ __attribute__((aligned(256))) uint8_t pad_lds[ONE ? 256 : 4];
    // copy instructions per wave and K-step when padded (ONE)
    constexpr int kCopiesPerStep = G::JA + G::JB + G::KSA + G::KSB;
    static_assert(!ONE || (CH - 1) * kCopiesPerStep <= 63, "outstanding copies must fit vmcnt");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
    const int wk = wave / NWG, wl = wave % NWG;                  // K group, wave in the group
    const int wm = wl / WGN, wn = wl % WGN;
    const int lr = lane & (MW - 1);         // row / column of the lane in a block
    const int lq = lane / MW;               // lane group

    // one work item per work-group (the dispatcher does the load balancing;
    // a persistent loop would hold the epilogue's per-lane address terms in
    // registers across the K loop)
    const int w = remap_block(blockIdx.x, gridDim.x);
    if (w >= p.total_work)
        return;
    {
        const TileCoord tc = decode_work(w, p.tiles_m, p.tiles_n, p.split, p.group_n);
        const int m0 = tc.tm * BM, n0 = tc.tn * BN;
        CopyOffsets<BM, BN, NWG, MW> co;
        copy_offsets(p, m0, n0, wl, lane, co);
        const int seg0 = tc.ks * p.segs_per_split;
        // the group's K-steps: s -> work-item K-step WGK s + wk
        const int nsteps = p.segs_per_split * (p.kpr / kBK) / WGK;
        auto src_of = [&](int s) { return step_src(p, seg0, n0, WGK * s + wk); };

        acc_t acc[GA][GB];
        // exact mode: running totals; each pair of K-steps is summed in
        // fresh accumulators first (see mxgemm_exact_kernel)
        acc_t tot[EXACT ? GA : 1][EXACT ? GB : 1];
#pragma unroll
        for (int i = 0; i < GA; ++i)
#pragma unroll
            for (int j = 0; j < GB; ++j)
#pragma unroll
                for (int v = 0; v < NACC; ++v) {
                    acc[i][j][v] = 0.f;
                    if constexpr (EXACT)
                        tot[i][j][v] = 0.f;
                }

        const int nsup = (nsteps + CH - 1) / CH;    // stages of CH K-steps
#pragma unroll
        for (int c = 0; c < CH; ++c)
            if (c < nsteps)
                copy_issue(co, src_of(c), stage0 + (c * WGK + wk) * G::STAGE, wl, 0, 1,
                           ONE ? pad_lds : nullptr);
        if (!ONE) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }

        // One stage: start the copies of stage t + 1 into NXT, multiply the
        // K-steps in CUR, then wait for the copies and synchronise.
        auto kstage = [&](int t, const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt) {
#pragma unroll
            for (int c = 0; c < CH; ++c)
                if (!ONE && (t + 1) * CH + c < nsteps)
                    copy_issue(co, src_of((t + 1) * CH + c), nxt + (c * WGK + wk) * G::STAGE, wl);
#pragma unroll
            for (int c = 0; c < CH; ++c) {
            if (t * CH + c >= nsteps)
                break;
            if constexpr (ONE) {
                // all copies were issued up front, in step order: K-step c
                // has landed once at most (nsteps - 1 - c) steps' copies
                // are outstanding
                wait_steps<kCopiesPerStep, CH - 1>(nsteps - 1 - c);
                __syncthreads();
            }
            const uint8_t* sub = cur + (c * WGK + wk) * G::STAGE;
            // Row r of a fragment group is r = group base + lr with the
            // group base a multiple of MW >= 16, so the swizzle key of r
            // equals that of lr: a lane's swizzled byte offsets differ
            // between groups by a constant.
            const uint8_t* pa = sub + (wm * TM + lr) * kBK;
            const uint8_t* pb = sub + G::A_BYTES + (wn * TN + lr) * kBK;
            const uint8_t* psa = sub + G::SA_OFF + (wm * TM + lr) * 4;
            const uint8_t* psb = sub + G::SB_OFF + (wn * TN + lr) * 4;
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
                            bf[j], af[cur], acc[i][j], FB, FA, 0, sbv[j], 0, sav[cur]);
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
                                bf[j][m], af[cur][m], acc[i][j], FB, FA, 0, sbv[j][m], 0, sav[cur][m]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                // Exact, 16 x 16 x 32 bf16, four MFMAs per (A group, B
                // group) per K-step: MFMA m (0, 1) of half s (0, 1) takes,
                // in lane group q = lane / 16, the codes of K [64s + 16q +
                // 8m, +8).  So one 16-byte read of logical chunk 4s + q
                // feeds both MFMAs of a half, and a read instruction's
                // lanes of rows 0..7 land on eight different 16-byte bank
                // groups (8-byte reads of two rows 8 apart share one).  A
                // and B use the same K assignment, so every product pairs
                // correctly; each lane folds in the scale of its own MX
                // block, 2s + q / 2.  Products are exact in the MFMA and
                // summed with FP32-grade precision.  Both halves' codes are
                // read first: one LDS round trip per K-step (these small
                // tiles have few MFMAs to hide latency behind).
                uint32_t sa_w[GA], sb_w[GB];
                u32x4 rb[2][GB], ra[2][GA];
                const int sshift = 8 * (lq >> 1);
#pragma unroll
                for (int g = 0; g < GB; ++g)
                    sb_w[g] = *reinterpret_cast<const uint32_t*>(psb + g * MW * 4) >> sshift;
#pragma unroll
                for (int i = 0; i < GA; ++i)
                    sa_w[i] = *reinterpret_cast<const uint32_t*>(psa + i * MW * 4) >> sshift;
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int lane_off = chunk(4 * s + lq);
#pragma unroll
                    for (int g = 0; g < GB; ++g)
                        rb[s][g] = *reinterpret_cast<const u32x4*>(pb + g * MW * kBK + lane_off);
#pragma unroll
                    for (int i = 0; i < GA; ++i)
                        ra[s][i] = *reinterpret_cast<const u32x4*>(pa + i * MW * kBK + lane_off);
                }
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        v8bf bb[GB], ab[GA];
#pragma unroll
                        for (int g = 0; g < GB; ++g)
                            bb[g] = fp8x8_to_bf16<FB>(m ? u32x2{rb[s][g].z, rb[s][g].w} : u32x2{rb[s][g].x, rb[s][g].y},
                                                      e8m0_to_f32(sb_w[g] >> (16 * s)));
#pragma unroll
                        for (int i = 0; i < GA; ++i)
                            ab[i] = fp8x8_to_bf16<FA>(m ? u32x2{ra[s][i].z, ra[s][i].w} : u32x2{ra[s][i].x, ra[s][i].y},
                                                      e8m0_to_f32(sa_w[i] >> (16 * s)));
#pragma unroll
                        for (int i = 0; i < GA; ++i)
#pragma unroll
                            for (int g = 0; g < GB; ++g)
                                acc[i][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bb[g], ab[i], acc[i][g], 0, 0, 0);
                    }
                // close the pair of K-steps that ends here (or the last step)
                const int step = t * CH + c;
                if ((step & 1) == 1 || step == nsteps - 1) {
#pragma unroll
                    for (int i = 0; i < GA; ++i)
#pragma unroll
                        for (int g = 0; g < GB; ++g) {
                            tot[i][g] += acc[i][g];
                            acc[i][g] = acc_t{};
                        }
                }
            }

            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        };
        for (int t = 0; t < nsup; t += 2) {
            kstage(t, stage0, stage1);
            if (t + 1 < nsup)
                kstage(t + 1, stage1, stage0);
        }

        if constexpr (WGK > 1) {
            // groups 1 .. WGK - 1 pass their sums through stage 0
            static_assert((WGK - 1) * NWG * TM * TN * 4 <= WGK * G::STAGE, "sums of the other groups fit a stage");
            reduce_k_groups<NWG, WGK, GA, GB>(acc, reinterpret_cast<float*>(stage0), wk, wl, lane);
        }
        if constexpr (!EXACT && MW == 32 && !ONE) {
            // Native large tiles: bfloat16 C as whole rows through LDS, as
            // in the exact kernel (the stages are free: every wave has
            // passed the last stage's barrier).  One K group: waves 0 ..
            // NW/2 - 1 use stage 0, the others stage 1; several: group 0
            // stores through stage 1 (stage 0 holds the other groups' sums).
            if (p.split == 1 && (reinterpret_cast<uintptr_t>(p.c) & 15) == 0 && (p.N & 7) == 0) {
                if constexpr (WGK == 1) {
                    static_assert(NW % 2 == 0 && (NW / 2) * TM * TN * 2 <= CH * G::STAGE,
                                  "half the wave tiles of bf16 per stage");
                    __syncthreads();
                    uint8_t* buf = (wave < NW / 2 ? stage0 : stage1) + (wave % (NW / 2)) * (TM * TN * 2);
                    store_tile_lds<GA, GB, TM, TN>(p, acc, buf, m0 + wm * TM, n0 + wn * TN, lane);
                } else {
                    static_assert(NWG * TM * TN * 2 <= WGK * G::STAGE, "bf16 wave tiles of one group fit a stage");
                    if (wk == 0)
                        store_tile_lds<GA, GB, TM, TN>(p, acc, stage1 + wl * (TM * TN * 2), m0 + wm * TM,
                                                       n0 + wn * TN, lane);
                }
                return;
            }
        }
        if (wk == 0) {
            if constexpr (EXACT)
                store_tile<GA, GB, MW>(p, tc, tot, m0 + wm * TM, n0 + wn * TN, lane);
            else
                store_tile<GA, GB, MW>(p, tc, acc, m0 + wm * TM, n0 + wn * TN, lane);
        }
        if (p.split > 1 && p.fused)
            split_combine<BM, BN>(p, tc, m0, n0);
    }
}

// Word e (0..7) of the bfloat16 operands of one 16-byte code piece: codes
// 2e, 2e + 1 (bytes of r in order) times sc.
template <int F>
__device__ __forceinline__ uint32_t cvt_word(const u32x4& r, float sc, int e)
{
    const uint32_t src = e < 2 ? r.x : e < 4 ? r.y : e < 6 ? r.z : r.w;
    return cvt2<F>(src, sc, (e & 1) != 0);
}

// Number of copies copy_issue(..., part, nparts) issues at most, and the
// t-th of them alone (same order), so the issue can be interleaved.
template <int BM, int BN, int NW, int MW>
__device__ __forceinline__ void copy_one(const CopyOffsets<BM, BN, NW, MW>& o, const StepSrc& src, uint8_t* dst,
                                         int wave, int part, int nparts, int t)
{
    typedef StageGeom<BM, BN, NW> G;
    int n = 0;
#pragma unroll
    for (int j = 0; j < G::JA; ++j)
        if (j % nparts == part && n++ == t && (G::IA % NW == 0 || wave + j * NW < G::IA))
            dma16_at(src.a, o.a[j], dst + (wave + j * NW) * 1024);
#pragma unroll
    for (int j = 0; j < G::JB; ++j)
        if (j % nparts == part && n++ == t && (G::IB % NW == 0 || wave + j * NW < G::IB))
            dma16_at(src.b, o.b[j], dst + G::A_BYTES + (wave + j * NW) * 1024);
#pragma unroll
    for (int j = 0; j < G::KSA; ++j)
        if (j % nparts == part && n++ == t && (G::ISA % NW == 0 || wave + j * NW < G::ISA))
            dma4_at(src.as, o.as[j], dst + G::SA_OFF + (wave + j * NW) * 256);
#pragma unroll
    for (int j = 0; j < G::KSB; ++j)
        if ((j + 1) % nparts == part && n++ == t && (G::ISB % NW == 0 || wave + j * NW < G::ISB))
            dma4_at(src.bs, o.bs[j], dst + G::SB_OFF + (wave + j * NW) * 256);
}

template <int BM, int BN, int NW>
__host__ __device__ constexpr int copies_in_part(int part, int nparts)
{
    typedef StageGeom<BM, BN, NW> G;
    int n = 0;
    for (int j = 0; j < G::JA; ++j)
        n += j % nparts == part;
    for (int j = 0; j < G::JB; ++j)
        n += j % nparts == part;
    for (int j = 0; j < G::KSA; ++j)
        n += j % nparts == part;
    for (int j = 0; j < G::KSB; ++j)
        n += (j + 1) % nparts == part;
    return n;
}

// Exact block-scaled GEMM on v_mfma_f32_32x32x16_bf16, software-pipelined.
//
// Accumulation: the MFMA adds its products into the FP32 accumulator in
// groups of eight with one round-to-nearest per group (measured: this
// model reproduces the kernel's outputs bit for bit).  Once a large
// product has entered an accumulator, every later group is rounded at that
// magnitude, so on data with outliers (products of 1e4 and more) an output
// that cancels to near zero collects errors of ~1e-2 over K = 8192.  So
// each pair of K-steps (256 K) is summed in fresh accumulators -- its first
// MFMAs take a zero accumulator input -- and then added to FP32 running
// totals: an output's roundings at large magnitude are then at most the 32
// of one pair plus one per pair.  The totals double the accumulator
// registers, which limits a wave to 128 x 64 outputs.
//
// WGM x WGN waves of (BM / WGM) x (BN / WGN), OCC per SIMD; large wave
// tiles keep the conversion work per MFMA low (each code a wave reads feeds
// BN / WGN resp. BM / WGM outputs).  A K-step (128 K) is four sub-steps of
// one MX block (32 K).  Lane group h = lane / 32 takes K [32j + 16h + 8m,
// +8) in MFMA m = 0, 1 of sub-step j, the same assignment for A and B, so
// one 16-byte read of logical chunk 2j + h feeds both MFMAs.
//
// Pipeline, per fragment (32 rows of A or B): while the MFMAs of sub-step j
// run, the fragment's codes of sub-step j + 1 (already in registers) are
// converted to bfloat16 with the block scale folded in (exact), and its
// codes of sub-step j + 2 are read from LDS into the freed registers.  A
// fragments are converted in place right after the MFMA group that used
// them; B fragments, used by every group, are double-buffered.  The one
// barrier of a K-step sits at sub-step 2: after it the copy of step s + 2
// reuses the stage just finished, and sub-steps 2 and 3 read the first
// codes of step s + 1.  The MFMAs take the B fragment as their first
// operand, so a lane's accumulators hold four consecutive columns of C.
//
// K groups (WGK > 1): WGK groups of WGM x WGN waves share the tile, group k
// taking K-steps k, k + WGK, k + 2 WGK, ... of the work item, so a small
// tile still gets large wave tiles (few conversions per MFMA) and enough
// waves.  A stage then holds WGK K-steps, one per group, each copied by its
// own group; every wave runs the pipeline above on its group's K-steps
// (pairs of them summed fresh).  At the end groups 1 .. WGK - 1 pass their
// totals through LDS and group 0 adds them in group order and stores the
// tile.  The work item's K-steps must be a multiple of WGK.
template <int BM, int BN, int WGM, int WGN, int WGK, int OCC, int FA, int FB>
__global__ void __launch_bounds__(WGM * WGN * WGK * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
mxgemm_exact_kernel(GemmArgs p)
{
    constexpr int MW = 32;
    constexpr int NWG = WGM * WGN;         // waves of one K group
    constexpr int NW = NWG * WGK;
    constexpr int TM = BM / WGM, TN = BN / WGN;
    constexpr int GA = TM / MW, GB = TN / MW;
    constexpr int NF = GA + GB;            // fragments a wave reads per sub-step
    static_assert(TM % MW == 0 && TN % MW == 0, "wave tile must be a multiple of the MFMA width");
    static_assert(GB <= GA && GA % GB == 0, "B fragments are spread evenly over the A groups");
    static_assert(GA * GB <= 8, "fresh and running accumulators of at most 128 x 64 outputs per wave");
    // upper bound of the work slices of one MFMA group (see kstep)
    constexpr int kMaxTasks = 20 + StageGeom<BM, BN, NWG>::JA + StageGeom<BM, BN, NWG>::JB + 4 + 2;
    typedef StageGeom<BM, BN, NWG> G;      // one K-step, copied by one K group

    __shared__ __attribute__((aligned(1024))) uint8_t stage0[WGK * G::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[WGK * G::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
    const int wk = wave / NWG, wl = wave % NWG;                  // K group, wave in the group
    const int wm = wl / WGN, wn = wl % WGN;
    const int lr = lane & 31, lq = lane >> 5;
    const int ksub = wk * G::STAGE;        // the group's K-step within a stage

    // Byte offsets in a stage of the lane's first A and B fragment rows and
    // of their scale words; fragment bases are multiples of 32 rows, so the
    // swizzle key of every row is that of lr.
    const int a_row = ksub + (wm * TM + lr) * kBK;
    const int b_row = ksub + G::A_BYTES + (wn * TN + lr) * kBK;
    const int sa_row = ksub + G::SA_OFF + (wm * TM + lr) * 4;
    const int sb_row = ksub + G::SB_OFF + (wn * TN + lr) * 4;
    auto frag_off = [&](int f) { return f < GA ? a_row + f * MW * kBK : b_row + (f - GA) * MW * kBK; };
    auto scale_off = [&](int f) { return f < GA ? sa_row + f * MW * 4 : sb_row + (f - GA) * MW * 4; };
    auto chunk_off = [&](int j) { return swz_t<MW>(lr, 2 * j + lq) * 16; };

    // one work item per work-group (the dispatcher does the load balancing;
    // a persistent loop would hold the epilogue's per-lane address terms in
    // registers across the K loop)
    const int w = remap_block(blockIdx.x, gridDim.x);
    if (w >= p.total_work)
        return;
    {
        const TileCoord tc = decode_work(w, p.tiles_m, p.tiles_n, p.split, p.group_n);
        const int m0 = tc.tm * BM, n0 = tc.tn * BN;
        CopyOffsets<BM, BN, NWG, MW> co;
        copy_offsets(p, m0, n0, wl, lane, co);
        const int seg0 = tc.ks * p.segs_per_split;
        // the group's K-steps: s -> work-item K-step WGK s + wk
        const int nsteps = p.segs_per_split * (p.kpr / kBK) / WGK;
        auto src_of = [&](int s) { return step_src(p, seg0, n0, WGK * s + wk); };

        v16f acc[GA][GB];          // MFMA accumulators of the current pair of K-steps
        v16f tot[GA][GB];          // running totals of the finished pairs
#pragma unroll
        for (int i = 0; i < GA; ++i)
#pragma unroll
            for (int g = 0; g < GB; ++g)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    acc[i][g][v] = 0.f;
                    tot[i][g][v] = 0.f;
                }
        auto flush = [&]() {
#pragma unroll
            for (int i = 0; i < GA; ++i)
#pragma unroll
                for (int g = 0; g < GB; ++g)
                    tot[i][g] += acc[i][g];
        };

        u32x4 raw[NF];             // codes of the sub-step after the next
        u32x4 cva[GA][2];          // A operands (bfloat16 pairs) of the current sub-step
        u32x4 cvb[2][GB][2];       // B operands, by sub-step parity
        uint32_t sw[NF];           // scale words (4 MX blocks) of a K-step

        copy_issue(co, src_of(0), stage0 + ksub, wl);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (nsteps > 1)
            copy_issue(co, src_of(1), stage1 + ksub, wl);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            sw[f] = *reinterpret_cast<const uint32_t*>(stage0 + scale_off(f));
            raw[f] = *reinterpret_cast<const u32x4*>(stage0 + frag_off(f) + chunk_off(0));
        }
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const float sc = e8m0_to_f32(sw[f]);
            u32x4(&dst)[2] = f < GA ? cva[f] : cvb[0][f - GA];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                dst[e >> 2][e & 3] = f < GA ? cvt_word<FA>(raw[f], sc, e) : cvt_word<FB>(raw[f], sc, e);
            raw[f] = *reinterpret_cast<const u32x4*>(stage0 + frag_off(f) + chunk_off(1));
        }

        // Group i of a sub-step: the 2 GB MFMAs of A fragment i, each
        // followed by a slice of the group's other work, in this order:
        //   A fragment i: scale, 8 conversions (next sub-step), LDS read
        //     (the sub-step after);
        //   the B fragments assigned to group i: the same;
        //   at sub-step 2: this group's share of the copies of step s + 2,
        //     and the scale words of step s + 1 for fragments f = i mod GA.
        // sched_barrier fences keep that order, so the conversions run in
        // the MFMAs' shadow.
        // FRESH: the first K-step of a pair, whose first MFMA per output
        // block starts from a zero accumulator.
        auto kstep = [&](auto fresh, int s, const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt) {
            constexpr bool FRESH = decltype(fresh)::value;
            // Past the last K-step the copies repeat the last one (into the
            // stage just released, never read again): no branches here.
            const StepSrc src2 = src_of(s + 2 < nsteps ? s + 2 : nsteps - 1);
            uint32_t swn[NF];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = j & 1;
                if (j == 2) {
                    // every wave has read all of CUR and has its copies of
                    // step s + 1 in NXT
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    __syncthreads();
                }
                // Sub-steps j + 1, j + 2 are converted and read even past
                // the last K-step (then from the idle stage NXT; the values
                // are never used), which keeps this code branch-free.
                const uint8_t* src = j < 2 ? cur : nxt;
                const int coff = chunk_off((j + 2) & 3);
                const int jn = (j + 1) & 3;
#pragma unroll
                for (int i = 0; i < GA; ++i) {
                    constexpr int NU = 2 * GB;                        // MFMAs in the group
                    constexpr int RB = GA / GB;                       // groups per B fragment
                    const int nbf = i % RB == 0 ? 1 : 0;              // B fragment i / RB is the group's
                    const int gb = i / RB;
                    const int ncopy = j == 2 ? copies_in_part<BM, BN, NWG>(i, GA) : 0;
                    const int nsw = j == 2 ? 1 + (i + GA < NF ? 1 : 0) : 0;   // fragments i, i + GA
                    const int ntask = 10 * (1 + nbf) + ncopy + nsw;
                    u32x4 cva_n[2];
                    float sc = 0.f;
#pragma unroll
                    for (int u = 0; u < NU; ++u) {
                        const int m = u / GB, g = u % GB;
                        acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(v8bf, cvb[c][g][m]), __builtin_bit_cast(v8bf, cva[i][m]),
                            (FRESH && j == 0 && m == 0) ? v16f{} : acc[i][g], 0, 0, 0);
                        const int t0 = u * ntask / NU, t1 = (u + 1) * ntask / NU;
#pragma unroll
                        for (int t = 0; t < kMaxTasks; ++t) {
                            if (t < t0 || t >= t1)
                                continue;
                            if (t < 10) {                              // A fragment i
                                if (t == 0)
                                    sc = e8m0_to_f32(sw[i] >> (8 * jn));
                                else if (t < 9)
                                    cva_n[(t - 1) >> 2][(t - 1) & 3] = cvt_word<FA>(raw[i], sc, t - 1);
                                else
                                    raw[i] = *reinterpret_cast<const u32x4*>(src + frag_off(i) + coff);
                            } else if (t < 10 * (1 + nbf)) {           // B fragment gb
                                const int tb = t - 10;
                                if (tb == 0)
                                    sc = e8m0_to_f32(sw[GA + gb] >> (8 * jn));
                                else if (tb < 9)
                                    cvb[c ^ 1][gb][(tb - 1) >> 2][(tb - 1) & 3] = cvt_word<FB>(raw[GA + gb], sc, tb - 1);
                                else
                                    raw[GA + gb] = *reinterpret_cast<const u32x4*>(src + frag_off(GA + gb) + coff);
                            } else if (t < 10 * (1 + nbf) + ncopy) {   // copies of step s + 2
                                copy_one(co, src2, const_cast<uint8_t*>(cur) + ksub, wl, i, GA, t - 10 * (1 + nbf));
                            } else {                                   // scale words of step s + 1
                                const int f2 = i + GA * (t - 10 * (1 + nbf) - ncopy);
                                swn[f2] = *reinterpret_cast<const uint32_t*>(nxt + scale_off(f2));
                            }
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    cva[i][0] = cva_n[0];
                    cva[i][1] = cva_n[1];
                }
                if (j == 2) {
#pragma unroll
                    for (int f = 0; f < NF; ++f)
                        sw[f] = swn[f];
                }
            }
        };
        int s = 0;
        for (; s + 1 < nsteps; s += 2) {
            kstep(std::true_type(), s, stage0, stage1);
            kstep(std::false_type(), s + 1, stage1, stage0);
            flush();
        }
        if (s < nsteps) {
            kstep(std::true_type(), s, stage0, stage1);
            flush();
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy outlives the work-group

        if constexpr (WGK > 1) {
            // groups 1 .. WGK - 1 pass their totals through stage 0
            static_assert((WGK - 1) * NWG * TM * TN * 4 <= WGK * G::STAGE, "totals of the other groups fit a stage");
            reduce_k_groups<NWG, WGK, GA, GB>(tot, reinterpret_cast<float*>(stage0), wk, wl, lane);
        }
        if (p.split == 1 && (reinterpret_cast<uintptr_t>(p.c) & 15) == 0 && (p.N & 7) == 0) {
            // bfloat16 C through LDS: both stages are free once every wave
            // has passed this barrier (its copies landed, its reads done).
            // One K group: waves 0 .. NW/2 - 1 use stage 0, the others stage
            // 1; several: group 0 stores, through stage 1 (stage 0 holds the
            // other groups' totals, read until now).
            if constexpr (WGK == 1) {
                static_assert(NW % 2 == 0 && (NW / 2) * TM * TN * 2 <= G::STAGE, "half the wave tiles of bf16 per stage");
                __syncthreads();
                uint8_t* buf = (wave < NW / 2 ? stage0 : stage1) + (wave % (NW / 2)) * (TM * TN * 2);
                store_tile_lds<GA, GB, TM, TN>(p, tot, buf, m0 + wm * TM, n0 + wn * TN, lane);
            } else {
                static_assert(NWG * TM * TN * 2 <= WGK * G::STAGE, "bf16 wave tiles of one group fit a stage");
                if (wk == 0)
                    store_tile_lds<GA, GB, TM, TN>(p, tot, stage1 + wl * (TM * TN * 2), m0 + wm * TM,
                                                   n0 + wn * TN, lane);
            }
        } else {
            if (wk == 0)
                store_tile<GA, GB, MW>(p, tc, tot, m0 + wm * TM, n0 + wn * TN, lane);
            if (p.split > 1 && p.fused)
                split_combine<BM, BN>(p, tc, m0, n0);
        }
    }
}

template <int BM, int BN, int WGM, int WGN, int OCC, int MW, int CH, bool ONE, int FA, int FB>
static hipError_t launch_cfg(const GemmArgs& a, bool exact, hipStream_t stream)
{
    if (exact)
        hipLaunchKernelGGL((mxgemm_kernel<BM, BN, WGM, WGN, OCC, true, MW, CH, ONE, FA, FB>), dim3(a.total_work),
                           dim3(WGM * WGN * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((mxgemm_kernel<BM, BN, WGM, WGN, OCC, false, MW, CH, ONE, FA, FB>), dim3(a.total_work),
                           dim3(WGM * WGN * 64), 0, stream, a);
    return hipGetLastError();
}

// Large tiles: native on the scaled MFMA kernel (NWM x NWN waves), exact on
// the pipelined bf16 kernel (EWM x EWN waves, EWM * EWN / 4 per SIMD).
template <int BM, int BN, int NWM, int NWN, int NOCC, int EWM, int EWN, int FA, int FB>
static hipError_t launch_large(const GemmArgs& a, bool exact, hipStream_t stream)
{
    if (exact) {
        if constexpr ((BM / EWM) * (BN / EWN) <= 128 * 64) {
            // EWM x EWN waves, EWM * EWN / 4 per SIMD
            hipLaunchKernelGGL((mxgemm_exact_kernel<BM, BN, EWM, EWN, 1, EWM * EWN / 4, FA, FB>), dim3(a.total_work),
                               dim3(EWM * EWN * 64), 0, stream, a);
            return hipGetLastError();
        } else {
            // no exact-mode kernel: the fresh and running accumulators of a
            // 128 x 128 wave tile would not fit the register file (the
            // planner never asks for it)
            return hipErrorInvalidValue;
        }
    }
    hipLaunchKernelGGL((mxgemm_kernel<BM, BN, NWM, NWN, NOCC, false, 32, 1, false, FA, FB>),
                       dim3(a.total_work), dim3(NWM * NWN * 64), 0, stream, a);
    return hipGetLastError();
}

// The GEMM of tile configuration cfg (the host table's index) for A codes
// of format FA and B codes of format FB.
template <int FA, int FB>
hipError_t launch_gemm_fmt(int cfg, bool exact, const GemmArgs& a, hipStream_t stream)
{
    switch (cfg) {
    case 0: return launch_large<256, 256, 2, 4, 2, 2, 2, FA, FB>(a, exact, stream);
    case 1: return launch_large<256, 128, 2, 2, 1, 4, 2, FA, FB>(a, exact, stream);
    case 2: return launch_large<128, 128, 2, 2, 1, 2, 2, FA, FB>(a, exact, stream);
    case 3: return launch_cfg<64, 64, 2, 2, 2, 16, 2, false, FA, FB>(a, exact, stream);
    case 4: return launch_cfg<32, 64, 1, 4, 2, 16, 3, false, FA, FB>(a, exact, stream);
    case 5: return launch_cfg<16, 64, 1, 4, 2, 16, 3, false, FA, FB>(a, exact, stream);
    case 6: return launch_cfg<32, 64, 1, 4, 1, 16, kOneShotSteps, true, FA, FB>(a, exact, stream);
    case 7:
        // 64 x 64 in four K groups of one 64 x 64 wave
        if (a.segs_per_split * (a.kpr / kBK) % 4 != 0)
            return hipErrorInvalidValue;
        if (exact)
            hipLaunchKernelGGL((mxgemm_exact_kernel<64, 64, 1, 1, 4, 1, FA, FB>), dim3(a.total_work), dim3(256), 0,
                               stream, a);
        else
            hipLaunchKernelGGL((mxgemm_kernel<64, 64, 1, 1, 1, false, 32, 1, false, FA, FB, 4>), dim3(a.total_work),
                               dim3(256), 0, stream, a);
        return hipGetLastError();
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mxg
