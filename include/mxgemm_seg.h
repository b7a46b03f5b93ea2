/*
 * mxgemm_seg -- segmented MXFP8 GEMM for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Only plain integers and pointers cross it; device pointers are HIP
 * device addresses, `stream` is a hipStream_t passed as void* (NULL = the
 * default stream).  Every entry point returns MXGEMM_OK (0) or a negative
 * error code; mxgemm_seg_last_error() then gives a message for the calling
 * thread.  No entry point aborts the process.
 *
 * The operation is the compute half of a fused all-to-all + MXFP8 matmul
 * (cannbot-harness 0.1.5 package diff, all_to_all_matmul_impl.h: the
 * all-to-all/matmul class and its E4M3E4M3 kernel entry; all_to_all_matmul.cpp:
 * problem statement `m k n rankNum`, headMSize = rows per communication
 * chunk, bufferSize = pipeline depth).  Each of R ranks holds A as R segments
 * of [M, kPerRank]; segment r arrives from source rank r in chunks of
 * commMSize rows into a ring of `buffer_count` staging buffers, and the GEMM
 * consumes the chunks that have arrived:
 *
 *   C[m, n] = sum_{r<R} sum_{k<kPerRank} A_r[m, k] * B[n, r*kPerRank + k]
 *
 * with every operand MXFP8: FP8 codes (E4M3, OCP "FN", by default; E5M2 on
 * request, per operand) plus one E8M0 scale byte per 32 consecutive
 * K-elements, value = fp8(q) * 2^(scale - 127).
 * Products accumulate in FP32 over all segments (all_to_all_matmul_impl.h,
 * SetupParams: splitKNum = rankSize) and C is written as bfloat16 with
 * round-to-nearest-even.  On one GPU the R ranks are simulated: all R
 * segments live in this GPU's memory and a staging kernel stands in for the
 * all-to-all put.
 */
#ifndef MXGEMM_SEG_H
#define MXGEMM_SEG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MXGEMM_OK = 0,
    MXGEMM_EINVAL = -1,        /* an argument breaks a documented rule      */
    MXGEMM_ENOMEM = -2,        /* device allocation failed                  */
    MXGEMM_EHIP = -3,          /* a HIP runtime call failed                 */
    MXGEMM_EUNSUPPORTED = -4,  /* valid, but not supported by this build or
                                  device (not gfx950, shape limits)         */
    MXGEMM_ETIMEOUT = -5       /* flags protocol: a device wait gave up     */
};

typedef struct mxgemm_seg* mxgemm_seg_t;

/* Arithmetic of the GEMM core.
 *  MXGEMM_PRECISION_EXACT (default): every FP8 x FP8 x 2^(scales) product
 *    is formed exactly (codes are converted to bfloat16 with the block scale
 *    folded in, which is exact for scale bytes >= 3 with E4M3 codes, >= 10
 *    with E5M2) and the products are summed on the bfloat16 MFMA
 *    (v_mfma_f32_32x32x16_bf16 on the 256 x 128, 128 x 128 and K-group
 *    64 x 64 tiles, v_mfma_f32_16x16x32_bf16 on the other small ones), which
 *    adds them into FP32 in groups of eight.  Each pair of K-steps (256 K)
 *    is summed in fresh accumulators and then added to FP32 running totals,
 *    so a large product rounds the small ones after it only until the pair
 *    ends.  The result is an FP32 sum in a fixed order, rounded once to
 *    bfloat16; like any FP32 sum it can lose small terms to cancellation of
 *    large ones (2^30 + 1 - 2^30 gives 0).  Tested: |C - exact| <= 1e-2 +
 *    8e-3 |exact| on every output of the five measured workloads without
 *    outliers and, on the 8192-cube outlier workload, on every output whose
 *    |C| is under 5% of the RMS plus 2^20 random ones; bit-exact results on
 *    integer-valued data whose sums stay below 2^8.  The 256 x 256 tile has
 *    no exact-mode kernel.
 *  MXGEMM_PRECISION_NATIVE: the CDNA4 block-scaled FP8 MFMA
 *    (v_mfma_scale_f32_32x32x64_f8f6f4 on the large tiles,
 *    v_mfma_scale_f32_16x16x128_f8f6f4 on the small ones) at twice the peak
 *    rate.  Its internal block dot drops products that are ~2^13 times
 *    smaller than another product of the same group of eight, so data with
 *    large in-block dynamic range (outliers) can miss the tolerance above
 *    where C is small; it meets it on the five workloads without outliers. */
enum { MXGEMM_PRECISION_EXACT = 0, MXGEMM_PRECISION_NATIVE = 1 };

/* FP8 formats of the A and B codes.  The pages ship four entries of the
 * same operator, one per (A, B) pair of E4M3 (OCP "FN") and E5M2 (OCP,
 * bias 15, infinities and NaNs, largest finite 57344):
 * all_to_all_matmul_impl.h, AllToAllQuantMatmulKernelE4M3E4M3, ...E5M2E5M2,
 * ...E4M3E5M2 and ...E5M2E4M3.  Scales are E8M0 per 32 K-elements in every
 * case.  Exact mode converts either format to bfloat16 exactly (E5M2 codes
 * need a scale byte >= 10 to stay on the bfloat16 grid, E4M3 codes >= 3);
 * native mode passes the formats to the scaled MFMA. */
enum { MXGEMM_FMT_E4M3 = 0, MXGEMM_FMT_E5M2 = 1 };

/* Ring protocols: how a GEMM learns that a chunk has landed in the ring
 * and the staging side that a slot may be refilled.  Both are on the
 * pages (all_to_all_matmul_impl.h, MatmulProcess / AllToAllProcess).
 *
 *  MXGEMM_RING_EVENTS: per window of W chunks, a staging kernel on the
 *    handle's side stream, a ready event, the GEMM launch (and a split-K
 *    sum) on the caller's stream, a credit event.
 *
 *  MXGEMM_RING_FLAGS: one persistent launch per run.  Work-group b keeps
 *    tile column b / S of C (64 columns) and K-split b % S for the whole
 *    run, holds its B tile (64 rows x the split's K range, at most 1024) in
 *    LDS, stages its share of every window into the ring, and hands over
 *    through counters in device memory: ready and credit per (slot group,
 *    split).  Everything one work-group writes for another (ring data,
 *    partials, counters) goes through device-scope stores and loads, and a
 *    count is raised only after the writer's stores have completed.  The
 *    last split to finish a tile sums the FP32 partials in split order.
 *    One launch and one read of B instead of one per window, for short M
 *    (skinny shapes); chosen only when asked for (options.ring), since the
 *    device-memory hand-overs made it slower than the events protocol on
 *    every measured shape.  Both precision modes.  All work-groups
 *    must be resident at once (at most one per compute unit); a wait that
 *    polls spin_limit times without progress gives up, marks the handle
 *    (mxgemm_seg_status) and lets the kernel finish, so a run never hangs.
 */
enum { MXGEMM_RING_EVENTS = 0, MXGEMM_RING_FLAGS = 1 };

/* Plan chosen for a problem: filled by mxgemm_seg_plan (host only, no GPU)
 * and by mxgemm_seg_get_plan for a live handle. */
typedef struct mxgemm_seg_plan {
    int64_t M, kPerRank, N, K, commMSize;
    int32_t rank_size, buffer_count;
    int32_t chunks;            /* ceil(M / commMSize)                       */
    int32_t chunks_per_window; /* W: chunks one stage/GEMM launch pair covers */
    int32_t windows;           /* ceil(chunks / W)                          */
    int32_t window_slots;      /* buffer_count / W ring windows             */
    int32_t tile_cfg;          /* index into the kernel tile table          */
    int32_t tile_m, tile_n;    /* output tile of one work-group             */
    int32_t split;             /* S: K split over rank-segment groups       */
    int32_t tiles_m, tiles_n;  /* tiles of a full window                    */
    int32_t work_items;        /* tiles_m * tiles_n * S for a full window   */
    int32_t grid;              /* work-groups of a full-window GEMM launch:
                                  one per work item                        */
    int32_t group_n;           /* N-tiles per zigzag group                  */
    int32_t num_cus;
    int32_t precision;         /* MXGEMM_PRECISION_*                        */
    int32_t a_format;          /* MXGEMM_FMT_* of the A codes               */
    int32_t b_format;          /* MXGEMM_FMT_* of the B codes               */
    int32_t ring;              /* MXGEMM_RING_*                             */
    int32_t spin_limit;        /* flags protocol: polls before a wait gives up */
    int32_t reserved;
    int64_t slot_bytes;        /* one staging buffer: R*commMSize*kPerRank  */
    int64_t scale_slot_bytes;  /* its scales: R*commMSize*kPerRank/32       */
    int64_t workspace_bytes;   /* FP32 split-K partials: S * W * commMSize * N * 4 */
} mxgemm_seg_plan_t;

/* Optional knobs for mxgemm_seg_create_ex / mxgemm_seg_plan; -1 = automatic.
 *
 * Tile table (tile_cfg: work-group tile of C, K-steps of 128 per LDS stage):
 *   0  256 x 256, 1 step   (native only: 8 waves)
 *   1  256 x 128, 1 step   (native: 4 waves of 128 x 64; exact: 8 of 64 x 64)
 *   2  128 x 128, 1 step   (exact: 4 waves of 64 x 64)
 *   3   64 x  64, 2 steps  (two work-groups per compute unit)
 *   4   32 x  64, 3 steps  (two per compute unit)
 *   5   16 x  64, 3 steps  (two per compute unit)
 *   6   32 x  64, one stage holding a work item's whole K range, at most 8
 *       steps ((rank_size / split) * kPerRank / 128 <= 8); planned only when
 *       asked for
 *   7   64 x  64: four waves of 64 x 64, each taking every fourth K-step
 *       of the work item, their sums added at the end; needs
 *       (rank_size / split) * kPerRank / 128 to be a multiple of 4
 * The planner picks the tile, split and window by a cost model; forcing a
 * value the problem cannot take fails with MXGEMM_EINVAL. */
typedef struct mxgemm_seg_options {
    int32_t tile_cfg;          /* force a tile configuration (table index)  */
    int32_t split;             /* force S (must divide rank_size)           */
    int32_t chunks_per_window; /* force W (must divide buffer_count)        */
    int32_t precision;         /* MXGEMM_PRECISION_* (-1 = EXACT)           */
    int32_t a_format;          /* MXGEMM_FMT_* of A (-1 = E4M3)             */
    int32_t b_format;          /* MXGEMM_FMT_* of B (-1 = E4M3)             */
    int32_t ring;              /* MXGEMM_RING_* (-1 = EVENTS)               */
    int32_t spin_limit;        /* flags protocol: polls per wait (-1 = ~1 s) */
} mxgemm_seg_options_t;

/*
 * Create a handle for one problem shape.
 *   M          rows of A and C                         (> 0)
 *   kPerRank   K columns per rank segment              (> 0, % 128 == 0)
 *   rank_size  R, number of (simulated) ranks          (1 .. 64)
 *   N          columns of C, rows of B ([N][K])        (> 0)
 *   commMSize  rows per staged chunk                   (> 0)
 *   buffer_count  staging ring depth                   (power of two, 1..64)
 * Rules follow all_to_all_matmul.cpp (argument parsing: positive sizes, K
 * divisible by rankNum) and all_to_all_matmul_impl.h (MatmulProcess: the
 * ring index is a bit mask, so the depth is a power of two).  There,
 * CalcMOffset / GetCurMSize size every chunk at commMSize rows, so rows past
 * the last whole chunk would be dropped; here the last chunk holds the
 * remaining M % commMSize rows when commMSize does not divide M.  The MX block is
 * 32; this build also needs kPerRank % 128 == 0 (one MFMA K-step), else
 * MXGEMM_EUNSUPPORTED.  Allocates, on the current device, the staging ring
 * (buffer_count * R * commMSize * kPerRank * 33/32 bytes), the split-K
 * workspace and its per-tile arrival counts, the flags protocol's counters,
 * a side stream at default priority and the ring's events; run() allocates
 * nothing.  Errors: EINVAL, ENOMEM, EHIP,
 * EUNSUPPORTED (device is not gfx950).  *out is set only on success.
 */
int mxgemm_seg_create(mxgemm_seg_t* out, int64_t M, int64_t kPerRank, int32_t rank_size,
                      int64_t N, int64_t commMSize, int32_t buffer_count);

/* As mxgemm_seg_create, with optional knobs (opts may be NULL): the tile,
 * split and window the source fixes in its tiling data (all_to_all_matmul.cpp,
 * GetTilingData over headMSize x n x ka; all_to_all_matmul_impl.h,
 * SetupParams), the operand formats of its four kernel entries, and the
 * ring protocol (MatmulProcess / AllToAllProcess).  Errors as create. */
int mxgemm_seg_create_ex(mxgemm_seg_t* out, int64_t M, int64_t kPerRank, int32_t rank_size,
                         int64_t N, int64_t commMSize, int32_t buffer_count,
                         const mxgemm_seg_options_t* opts);

/*
 * Enqueue one segmented GEMM on `stream`; returns once enqueued (no host
 * synchronisation).  All pointers are device memory, 16-byte aligned, owned
 * by the caller, and must stay valid until the work completes:
 *   a_seg    uint8 FP8   [R][M][kPerRank]     segment r is rank r's K range
 *   a_scale  uint8 E8M0  [R][M][kPerRank/32]
 *   b        uint8 FP8   [N][K], K = R*kPerRank, K contiguous (B transposed)
 * (FP8 codes in the plan's a_format / b_format, E4M3 by default)
 *   b_scale  uint8 E8M0  [N][K/32]
 *   c        bfloat16    [M][N], fully overwritten
 * A scale byte 0xFF (the E8M0 NaN) makes every output that takes a product
 * from its block NaN, in both precision modes.
 * Layouts: all_to_all_comm_udma.h, PutSegmentToRank / PutScaleToRank (source
 * offsets r*M*rowBytes + mOffset*rowBytes), all_to_all_matmul.cpp (host
 * buffer sizes), all_to_all_matmul_impl.h (TransB = true, C offset
 * mOffset * N).  Chunk j (rows [j*commMSize, min((j+1)*commMSize, M)) of every
 * segment, with their scales) is copied by a staging kernel into ring slot
 * j % buffer_count; the GEMM for a chunk starts only after its copy (ready)
 * and a slot is refilled only after the GEMM that read it (credit) -- the
 * ready/credit pairing of MatmulProcess / AllToAllProcess.  With two or
 * more slot groups (buffer_count / W >= 2) the staging runs ahead on the
 * handle's side stream, paired with the GEMMs by ready and credit events;
 * with one slot group it could not run ahead, and both kernels run in
 * order on `stream`.  With S > 1 a window's GEMM writes FP32
 * partials into the handle's workspace and they are summed in split order
 * into C (the result does not depend on timing): by the last split of each
 * tile to finish, inside the GEMM launch, when a tile's partials of all
 * splits take at most 128 KiB, else by a second kernel on `stream`.  The
 * side stream, when used, forks from and joins back into `stream`; with the
 * flags protocol everything is one launch on `stream`.  Work before and
 * after run() on `stream` therefore stays
 * ordered and the call can be captured into a HIP graph.  A handle must not
 * be run concurrently on two streams; distinct handles may.
 * Errors: EINVAL (NULL handle/pointer, misaligned pointer; a buffer the
 * GPU cannot access, i.e. host memory that is not pinned, or device memory
 * of another device), EHIP.  The accessibility check runs when the pointers
 * differ from the last ones that passed, and enqueues nothing.  Buffer
 * sizes are not checked: each buffer must hold the bytes stated above.
 */
int mxgemm_seg_run(mxgemm_seg_t h, const void* a_seg, const void* a_scale, const void* b,
                   const void* b_scale, void* c, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): one
 * segmented GEMM exactly as mxgemm_seg_run would do it for a handle created
 * with the same arguments and options, but with no handle and no
 * allocation.  The staging ring, the split-K workspace and the per-tile
 * arrival counts live in one static device array of 32 MiB per GPU, held
 * until the process ends; problems whose ring and workspace need more fail
 * with MXGEMM_EUNSUPPORTED (the five measured workloads need at most
 * 17.3 MB).  The staging always runs in order on `stream` (one window per
 * ring fill: no side stream, no events); options may be NULL, and
 * options.ring must be -1 or MXGEMM_RING_EVENTS, options.chunks_per_window
 * -1 or buffer_count.  Every call on one GPU uses that GPU's array and
 * leaves its contents behind: calls that overlap on one GPU (two streams,
 * two threads) race and give undefined C; calls in order on one stream are
 * safe.  The first call on a device looks up the array's address there.
 * Buffers and layouts as mxgemm_seg_run; asynchronous on `stream`.
 * Errors: EINVAL, EUNSUPPORTED, EHIP.
 */
int mxgemm_seg_run_static(int64_t M, int64_t kPerRank, int32_t rank_size, int64_t N,
                          int64_t commMSize, int32_t buffer_count, const mxgemm_seg_options_t* opts,
                          const void* a_seg, const void* a_scale, const void* b,
                          const void* b_scale, void* c, void* stream);

/*
 * Flags protocol (the device-flag hand-over of all_to_all_matmul_impl.h,
 * MatmulProcess waiting on the flag AllToAllProcess sets after a copy):
 * MXGEMM_ETIMEOUT if a device wait of any run since the last call gave up (the work-groups of a run were not all resident at
 * once, e.g. another kernel held compute units; C of such a run is
 * undefined), else MXGEMM_OK; clears the mark.  Waits for all work on the
 * device.  Always MXGEMM_OK for the events protocol.
 */
int mxgemm_seg_status(mxgemm_seg_t h);

/* Wait for the handle's work and free everything create() allocated: the
 * ring, the workspace and counters, the side stream and the events.  This is
 * the teardown at the end of the source's host run (all_to_all_matmul.cpp,
 * runAllToAllMatmul: device buffers freed, then the shared window and the
 * stream released).  NULL is accepted (nothing to free).  Errors: EHIP if
 * waiting for the work failed; every resource is still released and the
 * handle must not be used again. */
int mxgemm_seg_destroy(mxgemm_seg_t h);

/* Message for the last failing call on the calling thread ("" if none);
 * the string is owned by the library and valid until the thread's next
 * failing call.  The source reports errors the same two ways: a negative
 * return (all_to_all_matmul.cpp: parseArguments throws and main returns -1,
 * runAllToAllMatmul returns -1 when initialisation fails) and a message
 * (the exception text printed with the usage).  Never fails. */
const char* mxgemm_seg_last_error(void);

/* Copy the live handle's plan: the launch geometry the source computes on
 * the host before its launch (all_to_all_matmul.cpp, GetTilingData and
 * usedCoreNum as the launch's core count).  Errors: EINVAL (NULL). */
int mxgemm_seg_get_plan(mxgemm_seg_t h, mxgemm_seg_plan_t* out);

/* Compute the plan create() would choose on a device with `num_cus` compute
 * units, without touching a GPU (same rules and errors as create; opts may
 * be NULL); the host-side tiling step of all_to_all_matmul.cpp
 * (GetTilingData) for this library's kernels. */
int mxgemm_seg_plan(mxgemm_seg_plan_t* out, int64_t M, int64_t kPerRank, int32_t rank_size,
                    int64_t N, int64_t commMSize, int32_t buffer_count, int32_t num_cus,
                    const mxgemm_seg_options_t* opts);

/* Decode work item `w` of a window with `rows` rows under `plan` into
 * (tile row, tile column, K-split index), exactly as the GEMM kernel does
 * (flattened work ID with zigzag N-groups; Triton-distributed-Ascend
 * performance guide, section 1.2 on flattening the work ID and section 1.4
 * on the zigzag swizzle).  Also returns the work item that work-group
 * `block` of that window's launch (one work-group per work item) takes
 * under the XCD-aware remap.  Host only.
 * Errors: EINVAL (w or block out of range). */
int mxgemm_seg_decode(const mxgemm_seg_plan_t* plan, int64_t rows, int32_t w, int32_t block,
                      int32_t* tile_m_idx, int32_t* tile_n_idx, int32_t* split_idx,
                      int32_t* first_work);

/*
 * MXFP8 quantiser: x is float32 device memory [rows][cols] with row stride
 * ld_x elements (cols % 32 == 0); writes codes q [rows][cols] (row stride
 * ld_q bytes) and scale bytes s [rows][cols/32] (row stride ld_s bytes).
 * Per block of 32 consecutive elements of a row: e = the smallest integer
 * with 448 * 2^e >= amax, clamped to [-127, 127] (amax = 0 gives -127),
 * s = e + 127, q = E4M3 round-to-nearest-even of x * 2^-e (sign of zero
 * kept).  The pages produce their MXFP8 inputs offline with a generator they
 * do not show (all_to_all_matmul.cpp header: gen_data.py); this is the rule
 * 2^ceil(log2(amax/448)) written out exactly.  Non-finite input: a block
 * holding a NaN gets scale byte 0xFF (the E8M0 NaN) and every code 0x7F; a
 * block holding an infinity (and no NaN) gets e = 127 (the clamp), its
 * infinities the largest finite code of their sign and its finite elements
 * the rule above.  Asynchronous on `stream`.  Errors: EINVAL, EHIP.
 */
int mxgemm_quantize_mxfp8(const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                          uint8_t* q, int64_t ld_q, uint8_t* s, int64_t ld_s, void* stream);

/*
 * As mxgemm_quantize_mxfp8 for codes of `format` (MXGEMM_FMT_*), the input
 * formats of the source's sibling kernel entries (all_to_all_matmul_impl.h,
 * ...E5M2E5M2, ...E4M3E5M2, ...E5M2E4M3).  For E5M2
 * the rule uses its largest finite value: e = the smallest integer with
 * 57344 * 2^e >= amax, clamped to [-127, 127], and codes are E5M2
 * round-to-nearest-even of x * 2^-e, saturating at 57344 (MX conversions
 * saturate).  Errors: EINVAL (also for an unknown format, and for x, q or
 * s in memory the GPU cannot access, such as pageable host memory), EHIP.
 */
int mxgemm_quantize_mx(const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                       uint8_t* q, int64_t ld_q, uint8_t* s, int64_t ld_s, int32_t format,
                       void* stream);

/*
 * Kernel timing for measurement (the source's perf mode in
 * all_to_all_matmul.cpp times each kernel launch on its own, after a cache
 * flush, with a stream synchronisation per round).  While enabled, run()
 * brackets every GEMM
 * kernel launch (on `stream`; a separate split-K reduce kernel after it is
 * outside the bracket, a fused combine inside) and every staging launch
 * (on the stream it runs on) with timing events; the flags protocol's one
 * launch counts as a GEMM launch.  mxgemm_seg_kernel_times synchronises the handle and
 * returns the summed durations (ms) and launch counts since the last call,
 * then resets them.  Not for use under graph capture.  Errors: EINVAL, EHIP.
 */
int mxgemm_seg_set_profiling(mxgemm_seg_t h, int32_t enable);
int mxgemm_seg_kernel_times(mxgemm_seg_t h, double* gemm_ms, int32_t* gemm_launches,
                            double* stage_ms, int32_t* stage_launches);


#ifdef __cplusplus
}
#endif

#endif /* MXGEMM_SEG_H */
