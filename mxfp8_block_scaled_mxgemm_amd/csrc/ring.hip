// Device-flag variant of the ring: staging, ready/credit hand-over, the
// block-scaled GEMM and the split-K combine in one persistent launch.
//
// The pages describe this variant next to the event-paired one
// (all_to_all_matmul_impl.h, MatmulProcess / AllToAllProcess: the consumer
// waits on a per-chunk flag the producer sets after its copy, and the
// producer waits on a flag the consumer sets once a buffer may be reused).
// Here the roles live in the same work-groups:
//
//   work-group b: tile column tn = b / split, K-split s = b % split
//   (segments [s * sps, (s + 1) * sps)); the tiles_n work-groups with the
//   same s form split group s.
//
//   produce(w): wait until every member of the group has consumed the
//     window that last used the slot group (credit), copy this
//     work-group's share of window w's chunks of the group's segments into
//     the ring, then add 1 to ready[g][s] (release).
//   consume(w): wait for ready[g][s] to reach tiles_n per use of the slot
//     group (acquire), copy the window's rows of the group's segments from
//     the ring into LDS tile row by tile row, add 1 to credit[g][s] after
//     the last of them, multiply against the B tile held in LDS since the
//     start, and store.  With split > 1 each split writes an FP32 partial
//     and the last to arrive at a tile (a per-tile counter) sums the splits
//     in index order and writes C, so the result does not depend on timing.
//
// Coherence between work-groups on different XCDs (each XCD has its own
// L2): everything one work-group writes for another -- ring data, split-K
// partials, counters -- is written with device-scope stores (write-through
// to the memory side) and read with device-scope loads (which miss a stale
// L2 line), and a count is raised only after the writer's stores have
// completed (vmcnt(0)).  No agent-wide release or acquire fence is used:
// those write back or invalidate a whole L2, which costs microseconds when
// every work-group of an XCD does it for every window.
//
// Every wait polls at most spin_limit times; a wait that gives up sets
// *err and the work-group carries on, so every wave always reaches the
// end.  The last work-group to finish sets every counter back to zero for
// the next run.  A run needs all its work-groups resident at once (the host
// launches at most one per compute unit).
#include "device_util.h"

namespace mxg {
namespace {

constexpr int BM = kRingBM, BN = kRingBN, KS = kRingMaxSteps, NT = kRingThreads;
constexpr int A_STEP = BM * kBK, B_STEP = BN * kBK;   // LDS bytes per K-step

// Row length (floats) of the wave partials in LDS: 64 columns + 4 of pad,
// so the 16 rows a store instruction covers start on different banks.
constexpr int kRedRow = 68;

// Cache-policy operand of global_load_lds: SC1, device scope.
constexpr int kDeviceScope = 16;

// Thread 0 polls *ptr (device-scope loads) until it reaches `target` or
// gives up; the barrier holds the work-group until then, so its later
// device-scope loads see what the count's writers stored before raising it.
__device__ __forceinline__ void wait_geq(uint32_t* ptr, uint32_t target, const RingArgs& p)
{
    if (threadIdx.x == 0) {
        int n = 0;
        while (__hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (++n > p.spin_limit) {
                __hip_atomic_fetch_or(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
}

// Every thread's device-scope stores have completed (stores_done() in
// each thread, then a barrier): thread 0 raises the count.
__device__ __forceinline__ void signal(uint32_t* ptr)
{
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(ptr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// This work-group's share of window w (chunks [chunk0, chunk0 + nch)) of
// the group's segments: data in 16-byte and scales in 4-byte units.  Pair
// (chunk c, segment r) is one contiguous block of the source and of its
// ring slot (the layout of the event-paired staging kernel); the units of
// the group's pairs are dealt out over its tiles_n members, thread t of
// member tn taking units tn * 256 + t + i * tiles_n * 256.
struct StageGeo {
    int64_t upp, total;       // data units per pair, in the window
    int64_t upp_s, total_s;   // scale units per pair, in the window
};

__device__ __forceinline__ StageGeo stage_geo(const RingArgs& p, int nch)
{
    StageGeo g;
    g.upp = p.cms * p.kpr / 16;
    g.total = (int64_t)nch * p.segs_per_split * g.upp;
    g.upp_s = p.cms * (p.kpr >> 5) / 4;
    g.total_s = (int64_t)nch * p.segs_per_split * g.upp_s;
    return g;
}

// Source and ring offsets of data unit u (16 bytes) or scale unit u (4
// bytes); false for a unit past the rows of a short last chunk.
__device__ __forceinline__ bool unit_addr(const RingArgs& p, int chunk0, int seg0, int64_t u,
                                          int64_t upp, int64_t row_units, int64_t bytes_per_row,
                                          int64_t slot_bytes, int64_t unit, int64_t& src,
                                          int64_t& dst)
{
    const int sps = p.segs_per_split;
    const int64_t pair = u / upp, off = u - pair * upp;
    const int c = (int)(pair / sps), r = seg0 + (int)(pair % sps);
    const int64_t j = chunk0 + c;
    const int64_t left = p.M - j * p.cms;
    const int64_t rows = left < p.cms ? left : p.cms;
    src = ((int64_t)r * p.M + j * p.cms) * bytes_per_row + off * unit;
    dst = (j & (p.nbuf - 1)) * slot_bytes + (int64_t)r * p.cms * bytes_per_row + off * unit;
    return off < rows * row_units;
}

// The thread's first data and scale units, read before the slots are free.
struct StagePre {
    u32x4 v;
    uint32_t sv;
    int64_t dst, dst_s;
    bool has, has_s;
};

__device__ __forceinline__ StagePre stage_prefetch(const RingArgs& p, int chunk0, int nch, int seg0,
                                                   int tn)
{
    const StageGeo g = stage_geo(p, nch);
    const int64_t sk = p.kpr >> 5;
    const int64_t u = (int64_t)tn * NT + threadIdx.x;
    StagePre q;
    int64_t src;
    q.has = u < g.total &&
            unit_addr(p, chunk0, seg0, u, g.upp, p.kpr / 16, p.kpr, p.slot_bytes, 16, src, q.dst);
    if (q.has)
        q.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.a_seg + src));
    q.has_s = u < g.total_s &&
              unit_addr(p, chunk0, seg0, u, g.upp_s, sk / 4, sk, p.scale_slot_bytes, 4, src, q.dst_s);
    if (q.has_s)
        q.sv = *reinterpret_cast<const uint32_t*>(p.sa_seg + src);
    return q;
}

__device__ __forceinline__ void put16(uint8_t* dst, const u32x4& v) { st_dev16(dst, v); }

// Store the prefetched units, then copy the thread's remaining ones.
__device__ void stage_share(const RingArgs& p, int chunk0, int nch, int seg0, int tn,
                            const StagePre& q)
{
    const StageGeo g = stage_geo(p, nch);
    const int64_t sk = p.kpr >> 5;
    const int64_t stride = (int64_t)p.tiles_n * NT;
    const int64_t first = (int64_t)tn * NT + threadIdx.x;
    if (q.has)
        put16(p.ring + q.dst, q.v);
    if (q.has_s)
        st_dev(reinterpret_cast<uint32_t*>(p.sring + q.dst_s), q.sv);
    int64_t src, dst;
    for (int64_t u = first + stride; u < g.total; u += stride)
        if (unit_addr(p, chunk0, seg0, u, g.upp, p.kpr / 16, p.kpr, p.slot_bytes, 16, src, dst))
            put16(p.ring + dst, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.a_seg + src)));
    for (int64_t u = first + stride; u < g.total_s; u += stride)
        if (unit_addr(p, chunk0, seg0, u, g.upp_s, sk / 4, sk, p.scale_slot_bytes, 4, src, dst))
            st_dev(reinterpret_cast<uint32_t*>(p.sring + dst),
                   *reinterpret_cast<const uint32_t*>(p.sa_seg + src));
}

}  // namespace

template <int FA, int FB, bool EXACT>
__global__ void __launch_bounds__(NT) ring_kernel(RingArgs p)
{
    // LDS: the B tile for the whole run and one A tile, K-step by K-step
    // (128-byte rows, chunk position XOR-swizzled by row & 7), four scale
    // bytes per row and K-step (256-byte slots: one 64-lane copy), and the
    // four waves' FP32 partials of the tile.
    __shared__ __attribute__((aligned(1024))) uint8_t lds_b[KS * B_STEP];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_a[KS * A_STEP];
    __shared__ __attribute__((aligned(256))) uint8_t lds_sb[KS * 256];
    __shared__ __attribute__((aligned(256))) uint8_t lds_sa[KS * 256];
    __shared__ __attribute__((aligned(16))) uint8_t lds_red[4 * BM * kRedRow * 4];   // wave partials
    __shared__ uint32_t bcast;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lq = lane >> 4;

    const int s = blockIdx.x % p.split;
    const int tn = blockIdx.x / p.split;
    const int n0 = tn * BN;
    const int seg0 = s * p.segs_per_split;
    const int steps_per_seg = (int)(p.kpr / kBK);
    const int nsteps = p.segs_per_split * steps_per_seg;   // <= KS (host rule)
    const int64_t sk = p.kpr >> 5;
    const int K32 = p.K >> 5;

    uint32_t* ready = p.sync;
    uint32_t* credit = ready + p.window_slots * p.split;
    uint32_t* tile_cnt = credit + p.window_slots * p.split;
    uint32_t* done = tile_cnt + (int64_t)p.windows * p.tiles_m_win * p.tiles_n;

    // Staging of window w in two parts: the first loads (issued early)
    // and the rest (once the slots are free).
    auto produce_start = [&](int w) {
        const int chunk0 = w * p.W;
        const int nch = p.chunks - chunk0 < p.W ? p.chunks - chunk0 : p.W;
        return stage_prefetch(p, chunk0, nch, seg0, tn);
    };
    auto produce_finish = [&](int w, const StagePre& pre) {
        const int g = w % p.window_slots;
        const uint32_t use = (uint32_t)(w / p.window_slots);
        const int chunk0 = w * p.W;
        const int nch = p.chunks - chunk0 < p.W ? p.chunks - chunk0 : p.W;
        if (use > 0)
            wait_geq(credit + g * p.split + s, use * (uint32_t)p.tiles_n, p);
        stage_share(p, chunk0, nch, seg0, tn, pre);
        stores_done();
        __syncthreads();
        signal(ready + g * p.split + s);
    };
    auto produce = [&](int w) { produce_finish(w, produce_start(w)); };

    auto consume = [&](int w) {
        const int g = w % p.window_slots;
        const uint32_t use = (uint32_t)(w / p.window_slots);
        const int chunk0 = w * p.W;
        const int nch = p.chunks - chunk0 < p.W ? p.chunks - chunk0 : p.W;
        const int64_t row_base = (int64_t)chunk0 * p.cms;
        const int64_t left = p.M - row_base;
        const int rows_w = (int)((int64_t)nch * p.cms < left ? (int64_t)nch * p.cms : left);
        wait_geq(ready + g * p.split + s, (use + 1) * (uint32_t)p.tiles_n, p);

        const int tiles_m = (rows_w + BM - 1) / BM;
        for (int tm = 0; tm < tiles_m; ++tm) {
            // A rows [tm BM, tm BM + BM) of the window (the last valid row
            // repeated past the end; those results are not stored)
            {
                const int row = 8 * wave + (lane >> 3);        // wave: 8 rows
                int wr = tm * BM + row;
                wr = wr < rows_w ? wr : rows_w - 1;
                const int64_t j = chunk0 + wr / p.cms;
                const int64_t in = wr % p.cms;
                const uint8_t* base = p.ring + (j & (p.nbuf - 1)) * p.slot_bytes + in * p.kpr +
                                      swz(row, lane & 7) * 16;
                int srow = lane < BM ? lane : BM - 1;          // scales: lane = row
                int swr = tm * BM + srow;
                swr = swr < rows_w ? swr : rows_w - 1;
                const int64_t sj = chunk0 + swr / p.cms;
                const uint8_t* sbase = p.sring + (sj & (p.nbuf - 1)) * p.scale_slot_bytes +
                                       (swr % p.cms) * sk;
                for (int ks = 0; ks < nsteps; ++ks) {
                    const int seg = seg0 + ks / steps_per_seg;
                    const int64_t kk = (int64_t)(ks % steps_per_seg) * kBK;
                    __builtin_amdgcn_global_load_lds(
                        base + (int64_t)seg * p.cms * p.kpr + kk,
                        (__attribute__((address_space(3))) void*)(lds_a + ks * A_STEP + wave * 1024),
                        16, 0, kDeviceScope);
                    if ((ks & 3) == wave)
                        __builtin_amdgcn_global_load_lds(
                            sbase + (int64_t)seg * p.cms * sk + (kk >> 5),
                            (__attribute__((address_space(3))) void*)(lds_sa + ks * 256), 4, 0,
                            kDeviceScope);
                }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tm == tiles_m - 1)
                signal(credit + g * p.split + s);   // the window's ring reads are done
            // One slot group: the next window is staged around this tile's
            // multiply -- its first loads before, the rest after (by then
            // every member has given its credit for this window).
            const bool stage_next = tm == tiles_m - 1 && p.window_slots == 1 && w + 1 < p.windows;
            StagePre pre_next;
            if (stage_next)
                pre_next = produce_start(w + 1);

            // Wave `wave` multiplies K-steps wave, wave + 4, ... over the
            // whole 32 x 64 tile (2 x 4 blocks of 16 x 16): every code is
            // converted once.  Exact MFMA path: MX block jb is one
            // v_mfma_f32_16x16x32_bf16; lane group q takes codes K
            // [32 jb + 8q, +8) of A and B, converted to bfloat16 with the
            // block's scale folded in.  Two accumulators per block (even /
            // odd MX block) so consecutive MFMAs do not wait for each other.
            v4f acc[2][4][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int gb = 0; gb < 4; ++gb)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        acc[i][gb][h] = v4f{0.f, 0.f, 0.f, 0.f};
            for (int ks = wave; ks < nsteps; ks += 4) {
                const uint8_t* pa = lds_a + ks * A_STEP + lr * kBK;
                const uint8_t* pb = lds_b + ks * B_STEP + lr * kBK;
                if constexpr (!EXACT) {
                    // Native: one v_mfma_scale_f32_16x16x128_f8f6f4 per block
                    // and K-step; lane group q holds K [16q, 16q + 16) and
                    // [64 + 16q, +16) (chunks q and q + 4) and the scale
                    // byte of MX block q.
                    const int off_lo = swz(lr, lq) * 16, off_hi = swz(lr, lq + 4) * 16;
                    v8i af[2], bf[4];
                    int sav[2], sbv[4];
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const u32x4 lo = *reinterpret_cast<const u32x4*>(pa + i * 16 * kBK + off_lo);
                        const u32x4 hi = *reinterpret_cast<const u32x4*>(pa + i * 16 * kBK + off_hi);
                        af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                        sav[i] = lds_sa[ks * 256 + (i * 16 + lr) * 4 + lq];
                    }
#pragma unroll
                    for (int gb = 0; gb < 4; ++gb) {
                        const u32x4 lo = *reinterpret_cast<const u32x4*>(pb + gb * 16 * kBK + off_lo);
                        const u32x4 hi = *reinterpret_cast<const u32x4*>(pb + gb * 16 * kBK + off_hi);
                        bf[gb] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                        sbv[gb] = lds_sb[ks * 256 + (gb * 16 + lr) * 4 + lq];
                    }
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int gb = 0; gb < 4; ++gb)
                            acc[i][gb][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                bf[gb], af[i], acc[i][gb][0], FB, FA, 0, sbv[gb], 0, sav[i]);
                    continue;
                }
                uint32_t sa_w[2], sb_w[4];
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    sa_w[i] = *reinterpret_cast<const uint32_t*>(lds_sa + ks * 256 + (i * 16 + lr) * 4);
#pragma unroll
                for (int gb = 0; gb < 4; ++gb)
                    sb_w[gb] = *reinterpret_cast<const uint32_t*>(lds_sb + ks * 256 + (gb * 16 + lr) * 4);
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) {
                    const int off = swz(lr, 2 * jb + (lq >> 1)) * 16 + (lq & 1) * 8;
                    v8bf ab[2], bb[4];
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        ab[i] = fp8x8_to_bf16<FA>(*reinterpret_cast<const u32x2*>(pa + i * 16 * kBK + off),
                                                  e8m0_to_f32(sa_w[i] >> (8 * jb)));
#pragma unroll
                    for (int gb = 0; gb < 4; ++gb)
                        bb[gb] = fp8x8_to_bf16<FB>(*reinterpret_cast<const u32x2*>(pb + gb * 16 * kBK + off),
                                                   e8m0_to_f32(sb_w[gb] >> (8 * jb)));
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int gb = 0; gb < 4; ++gb)
                            acc[i][gb][jb & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                bb[gb], ab[i], acc[i][gb][jb & 1], 0, 0, 0);
                }
            }
            // Wave partials to LDS: element v of acc[i][gb] is row
            // 16 i + lr, column 16 gb + 4 lq + v of the tile (B was the
            // first MFMA operand); rows padded to 68 floats.
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int gb = 0; gb < 4; ++gb)
                    *reinterpret_cast<v4f*>(lds_red + ((wave * BM + i * 16 + lr) * kRedRow + gb * 16 + 4 * lq) * 4) =
                        acc[i][gb][0] + acc[i][gb][1];
            __syncthreads();
            // Thread t: tile row t / 8, columns 4 (t % 8) + 32 h, h = 0, 1
            // (eight lanes cover 128 contiguous bytes of a partial row per
            // store), the four waves' partials summed in wave order.
            const int orow = tid >> 3, ocol = (tid & 7) * 4;
            v4f o[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                o[h] = *reinterpret_cast<const v4f*>(lds_red + (orow * kRedRow + ocol + 32 * h) * 4);
#pragma unroll
                for (int wv = 1; wv < 4; ++wv) {
                    const v4f x = *reinterpret_cast<const v4f*>(
                        lds_red + ((wv * BM + orow) * kRedRow + ocol + 32 * h) * 4);
                    o[h][0] += x[0];
                    o[h][1] += x[1];
                    o[h][2] += x[2];
                    o[h][3] += x[3];
                }
            }
            if (stage_next)
                produce_finish(w + 1, pre_next);

            const int wr = tm * BM + orow;
            const int64_t grow = row_base + wr;
            const bool row_ok = wr < rows_w;
            if (p.split == 1) {
                if (row_ok) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int col = n0 + ocol + 32 * h;
                        uint16_t* cp = p.c + grow * p.N + col;
                        if (p.c_vec4 && col + 3 < p.N) {
                            *reinterpret_cast<u32x2*>(cp) = u32x2{pack_bf16x2(o[h][0], o[h][1]),
                                                                  pack_bf16x2(o[h][2], o[h][3])};
                        } else {
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                if (col + v < p.N)
                                    cp[v] = f32_to_bf16_rne(o[h][v]);
                        }
                    }
                }
            } else {
                float* wsp = p.ws + (int64_t)s * p.M * p.N;
                if (row_ok) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int col = n0 + ocol + 32 * h;
                        float* dp = wsp + grow * p.N + col;
                        if ((p.N & 3) == 0 && col + 3 < p.N) {
                            st_dev16(dp, __builtin_bit_cast(u32x4, o[h]));
                        } else {
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                if (col + v < p.N)
                                    st_dev(dp + v, o[h][v]);
                        }
                    }
                }
                stores_done();
                __syncthreads();
                if (tid == 0)
                    bcast = __hip_atomic_fetch_add(
                        tile_cnt + ((int64_t)w * p.tiles_m_win + tm) * p.tiles_n + tn, 1u,
                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __syncthreads();
                if (bcast == (uint32_t)(p.split - 1)) {
                    // last split of this tile: C = bf16(sum of the partials
                    // in split order)
                    const int nr = rows_w - tm * BM < BM ? rows_w - tm * BM : BM;
                    combine_tile(p.ws, p.M * p.N, p.c, row_base + tm * BM, nr, n0, BN, p.N,
                                 p.split, p.c_vec4 != 0);
                }
            }
            __syncthreads();   // the next tile row reuses lds_a
        }
    };

    // The B tile and its scales, once for the whole run (issued after the
    // first window's staging, whose loads would otherwise queue behind it).
    auto load_b = [&]() {
        for (int ks = 0; ks < nsteps; ++ks) {
            const int seg = seg0 + ks / steps_per_seg;
            const int64_t kk = (int64_t)seg * p.kpr + (int64_t)(ks % steps_per_seg) * kBK;
#pragma unroll
            for (int t = 0; t < BN / 8 / 4; ++t) {
                const int rg = wave + 4 * t;                   // group of 8 rows
                const int row = 8 * rg + (lane >> 3);
                const int gn = n0 + row < p.N ? n0 + row : p.N - 1;
                dma16(p.b + (int64_t)gn * p.K + kk + swz(row, lane & 7) * 16,
                      lds_b + ks * B_STEP + rg * 1024);
            }
            if ((ks & 3) == wave) {
                const int gn = n0 + lane < p.N ? n0 + lane : p.N - 1;   // BN = 64 = lanes
                dma4(p.bs + (int64_t)gn * K32 + (kk >> 5), lds_sb + ks * 256);
            }
        }
    };

    // Window order: with two or more slot groups, window w + 1 is staged
    // before window w is consumed (its credit only needs window
    // w + 1 - window_slots <= w - 1, consumed by every member in an earlier
    // iteration); with one slot group it is staged inside consume(w), right
    // after the credit for w (every member gives that credit once its ring
    // reads of w are done, which needs nothing but the staging of w).
    produce(0);
    load_b();
    for (int w = 0; w < p.windows; ++w) {
        if (p.window_slots > 1 && w + 1 < p.windows)
            produce(w + 1);
        consume(w);
    }

    // The last work-group to get here resets the counters for the next run
    // (every other work-group's counter updates have completed before its
    // `done` update).
    stores_done();
    __syncthreads();
    if (tid == 0) {
        const uint32_t n = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (n == gridDim.x - 1) {
            const int64_t words = ring_sync_words(p.window_slots, p.split, p.windows, p.tiles_m_win,
                                                  p.tiles_n);
            for (int64_t i = 0; i < words; ++i)
                __hip_atomic_store(p.sync + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <bool EXACT>
static hipError_t launch_ring_prec(const RingArgs& a, int fa, int fb, hipStream_t stream)
{
    const dim3 grid((unsigned)(a.tiles_n * a.split)), block(NT);
    if (fa == kE4M3 && fb == kE4M3)
        hipLaunchKernelGGL((ring_kernel<kE4M3, kE4M3, EXACT>), grid, block, 0, stream, a);
    else if (fa == kE5M2 && fb == kE5M2)
        hipLaunchKernelGGL((ring_kernel<kE5M2, kE5M2, EXACT>), grid, block, 0, stream, a);
    else if (fa == kE4M3 && fb == kE5M2)
        hipLaunchKernelGGL((ring_kernel<kE4M3, kE5M2, EXACT>), grid, block, 0, stream, a);
    else if (fa == kE5M2 && fb == kE4M3)
        hipLaunchKernelGGL((ring_kernel<kE5M2, kE4M3, EXACT>), grid, block, 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_ring(const RingArgs& a, int fa, int fb, bool exact, hipStream_t stream)
{
    return exact ? launch_ring_prec<true>(a, fa, fb, stream) : launch_ring_prec<false>(a, fa, fb, stream);
}

}  // namespace mxg
