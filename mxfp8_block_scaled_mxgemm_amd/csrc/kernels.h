// Internal interface between the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxg {

// One row of the GEMM tile table.
struct TileCfg {
    int tile_m, tile_n;     // output tile of one work-group
    int threads;            // work-group size (64-wide waves)
    int lds_bytes;          // LDS per work-group
    int blocks_per_cu;      // resident work-groups per compute unit
    float rel_rate;         // planner's relative MFMA efficiency estimate
    int steps_per_stage;    // K-steps of 128 copied per LDS stage
    bool exact;             // has an exact-mode kernel
    bool automatic;         // the planner may choose it unasked
    int k_groups;           // groups of waves splitting a work item's K-steps
                            // (their count must be a multiple of it)
    bool native;            // has a native-mode kernel
};

int num_tile_cfgs();
const TileCfg& tile_cfg(int i);
// Tile configuration whose work items copy their whole K range at once;
// usable only when a work item has at most kOneShotSteps K-steps of 128.
constexpr int kOneShotCfg = 6;
constexpr int kOneShotSteps = 8;

// Staging copy for one window: chunks [chunk0, chunk0 + nch) of every
// segment, data and scales, into ring slots chunk % nbuf.
struct StageArgs {
    const uint8_t* a_seg;     // [R][M][kpr]
    const uint8_t* sa_seg;    // [R][M][kpr/32]
    uint8_t* ring;            // [nbuf][R][cms][kpr]
    uint8_t* sring;           // [nbuf][R][cms][kpr/32]
    int64_t M, kpr, cms;
    int64_t slot_bytes, scale_slot_bytes;
    int R, chunk0, nch, nbuf;
};

// GEMM over one window of `rows` staged rows.
struct GemmArgs {
    const uint8_t* a;         // ring data of the window's first slot
    const uint8_t* as;        // ring scales of the window's first slot
    int64_t a_slot_stride;    // bytes between consecutive slots (data)
    int64_t as_slot_stride;   // bytes between consecutive slots (scales)
    const uint8_t* b;         // [N][K]
    const uint8_t* bs;        // [N][K/32]
    uint16_t* c;              // C + first window row * N
    float* ws;                // split-K partials [split][rows][N] (split > 1)
    uint32_t* tile_cnt;       // fused combine: arrivals per tile [tiles_m][tiles_n], zero between launches
    int fused;                // split > 1: the last split of a tile sums the partials
    int rows, N, K, kpr, cms;
    int tiles_m, tiles_n, split, segs_per_split, group_n, total_work;
    int c_vec4;               // C rows may be written 4 elements (8 bytes) at a time
};

// Split-K reduction: c[r][n] = bf16(sum over s in order of ws[s][r][n]).
struct ReduceArgs {
    const float* ws;
    uint16_t* c;
    int rows, N, split;
    int c_vec4;
};

struct QuantArgs {
    const float* x;
    uint8_t* q;
    uint8_t* s;
    int64_t rows, cols, ld_x, ld_q, ld_s;
    int fmt;                  // 0 = E4M3, 1 = E5M2
};

// Device-flag ring: one persistent launch per run.  Work-group b owns tile
// column b / split of C and K-split b % split for the whole run; it keeps
// its B tile (kRingBN rows x the split's K range) in LDS, stages its share
// of every window's chunks into the ring, and multiplies the window's rows
// once the other members of its split group have staged theirs.
constexpr int kRingBM = 32, kRingBN = 64;
constexpr int kRingMaxSteps = 8;          // K-steps of 128 per split (LDS)
constexpr int kRingThreads = 256;

struct RingArgs {
    const uint8_t* a_seg;     // [R][M][kpr]
    const uint8_t* sa_seg;    // [R][M][kpr/32]
    uint8_t* ring;            // [nbuf][R][cms][kpr]
    uint8_t* sring;           // [nbuf][R][cms][kpr/32]
    const uint8_t* b;         // [N][K]
    const uint8_t* bs;        // [N][K/32]
    uint16_t* c;              // [M][N]
    float* ws;                // split-K partials [split][M][N] (split > 1)
    uint32_t* sync;           // counters, zero between runs (ring_sync_words)
    uint32_t* err;            // set nonzero when a wait gives up
    int64_t M, kpr, cms, slot_bytes, scale_slot_bytes;
    int R, N, K, nbuf, chunks, W, windows, window_slots;
    int tiles_n, split, segs_per_split, tiles_m_win;
    int c_vec4;               // C rows may be written 4 elements at a time
    int spin_limit;           // polls before a wait gives up
};

// 32-bit counters a run of the flags protocol uses: ready and credit per
// (slot group, split), one per (window, tile row, tile column), and `done`.
__host__ __device__ inline int64_t ring_sync_words(int window_slots, int split, int windows, int tiles_m_win,
                               int tiles_n)
{
    return 2LL * window_slots * split + (int64_t)windows * tiles_m_win * tiles_n + 1;
}

hipError_t launch_ring(const RingArgs& a, int fa, int fb, bool exact, hipStream_t stream);

hipError_t launch_stage(const StageArgs& a, hipStream_t stream);
// One work-group per work item (a.total_work of them); fa, fb: the FP8
// formats of A and B (0 = E4M3, 1 = E5M2).
hipError_t launch_gemm(int cfg, bool exact, int fa, int fb, const GemmArgs& a, hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream);
hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
// p[0 .. n) = v
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t stream);

}  // namespace mxg
