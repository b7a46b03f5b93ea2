// Tile scheduler (flattened work ID, zigzag order, XCD remap) shared by the GEMM
// kernels and the host planner.
//
// One GEMM launch covers one window of staged chunks.  Its work is the set of
// (tile row, tile column, K-split) triples, flattened into one work ID so
// that the number of work items, not the number of tiles of one chunk, sets
// how many compute units are busy (Triton-distributed-Ascend performance
// guide, section 1.2: active cores = min(tasks, cores), fold more dimensions
// into the work ID until tasks >= cores).  Tiles are visited in N-groups of
// `group_n` columns, walking M forward on even groups and backward on odd
// ones, so the A rows used at the end of one group are the first ones the
// next group needs (section 1.4, zigzag traversal).  The K-split index is the
// fastest-varying part of the ID, so the splits of one tile run at the same
// time on neighbouring work-groups.
//
// Work-groups are dispatched round-robin over the XCDs (block b runs on XCD
// b % 8), and each XCD has its own L2.  The GEMM kernels run one work item
// per work-group; remap_block() gives the work-groups of one XCD a
// contiguous range of logical IDs, so the work-groups resident on an XCD at
// one time work on one compact patch of tiles.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MXG_HD __host__ __device__ __forceinline__
#else
#define MXG_HD inline
#endif

namespace mxg {

constexpr int kNumXcd = 8;

struct TileCoord {
    int tm, tn, ks;
};

// Logical starting work ID of block `b` in a grid of `g` blocks.
MXG_HD int remap_block(int b, int g)
{
    const int q = g / kNumXcd, rem = g % kNumXcd;
    const int x = b % kNumXcd, i = b / kNumXcd;
    return x * q + (x < rem ? x : rem) + i;
}

// Work ID -> tile coordinates.  tiles_m x tiles_n tiles, `split` K-splits,
// zigzag groups of `group_n` tile columns (the last group may be narrower).
MXG_HD TileCoord decode_work(int w, int tiles_m, int tiles_n, int split, int group_n)
{
    TileCoord c;
    c.ks = w % split;
    const int t = w / split;
    const int per_group = group_n * tiles_m;
    const int grp = t / per_group;
    const int within = t - grp * per_group;
    const int first_n = grp * group_n;
    const int left = tiles_n - first_n;
    const int gw = left < group_n ? left : group_n;
    int tm = within / gw;
    const int nn = within - tm * gw;
    if (grp & 1)
        tm = tiles_m - 1 - tm;
    c.tm = tm;
    c.tn = first_n + nn;
    return c;
}

}  // namespace mxg
