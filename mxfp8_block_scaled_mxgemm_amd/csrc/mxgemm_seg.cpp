// Host side of the segmented MXFP8 GEMM: argument rules, the launch plan,
// the staging ring with its ready/credit events, and the C ABI.
#include "mxgemm_seg.h"

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "schedule.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

// A failing HIP call is reported through the return code and the message;
// the thread's last HIP error is cleared so that a later, unrelated launch
// check does not report it again.
#define HIP_TRY(expr)                                                                   \
    do {                                                                                \
        hipError_t e_ = (expr);                                                         \
        if (e_ != hipSuccess) {                                                         \
            (void)hipGetLastError();                                                    \
            return fail(MXGEMM_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));    \
        }                                                                               \
    } while (0)

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Argument rules (see the header for their sources).
int validate(int64_t M, int64_t kpr, int32_t R, int64_t N, int64_t cms, int32_t nbuf)
{
    if (M <= 0 || kpr <= 0 || R <= 0 || N <= 0 || cms <= 0 || nbuf <= 0)
        return fail(MXGEMM_EINVAL, "all sizes must be positive (M=%lld kPerRank=%lld R=%d N=%lld "
                    "commMSize=%lld buffers=%d)", (long long)M, (long long)kpr, R, (long long)N,
                    (long long)cms, nbuf);
    if (R > 64)
        return fail(MXGEMM_EINVAL, "rank_size %d exceeds 64", R);
    if (!is_pow2(nbuf) || nbuf > 64)
        return fail(MXGEMM_EINVAL, "buffer_count %d must be a power of two in [1, 64]", nbuf);
    if (kpr % 32 != 0)
        return fail(MXGEMM_EINVAL, "kPerRank %lld must be a multiple of the MX block 32",
                    (long long)kpr);
    if (kpr % 128 != 0)
        return fail(MXGEMM_EUNSUPPORTED, "kPerRank %lld must be a multiple of 128 (one MFMA "
                    "K-step) in this build", (long long)kpr);
    const int64_t K = (int64_t)R * kpr;
    if (K > (1 << 22) || N >= (1LL << 31) || M >= (1LL << 31))
        return fail(MXGEMM_EUNSUPPORTED, "problem too large for 32-bit tile offsets");
    const int64_t ring = (int64_t)nbuf * R * cms * kpr;
    if (ring >= (1LL << 31))
        return fail(MXGEMM_EUNSUPPORTED, "staging ring of %lld bytes exceeds 2 GiB", (long long)ring);
    if (ceil_div(M, cms) > (1 << 30))
        return fail(MXGEMM_EUNSUPPORTED, "too many chunks");
    return MXGEMM_OK;
}

struct Choice {
    int cfg, split;
    double cost;
    int64_t work;   // work items of a full window
};

// Split-K combine inside the GEMM launch (the last split of a tile sums the
// partials) when one work-group's share is small: the tile's partials of
// all splits at most 128 KiB.  Larger tiles use a separate reduce kernel
// spread over the whole device.
bool fused_combine(int tile_m, int tile_n, int split)
{
    return split > 1 && (int64_t)tile_m * tile_n * split * 4 <= (128 << 10);
}

// Estimated time of one window under (cfg, split), in 2.4 GHz clocks.  A
// work item is bound either by its MFMAs (at the tile's efficiency, shared
// with the other resident work-groups of the CU) or by the round trips of
// its copy stages: a stage's copies are waited for before its K-steps
// start, and a round trip under load takes ~2 us.  The constants (the 1.6
// factor, 4400 clocks per copy round trip, 3000 per work item, 9000 per
// fused combine) were fitted on MI355X parts that ran these kernels at
// 1.84-2.2 GHz shader clock under load; the estimate ranks plans and does
// not predict times, and its units stay 2.4 GHz clocks whatever the clock.
double estimate(const mxg::TileCfg& t, int64_t rows, int64_t N, int64_t K, int split,
                int num_cus, bool exact)
{
    const int64_t tiles = ceil_div(rows, t.tile_m) * ceil_div(N, t.tile_n);
    const int64_t work = tiles * split;
    const int64_t cap = (int64_t)num_cus * t.blocks_per_cu;
    const int64_t rounds = ceil_div(work, cap);
    const double flops = 2.0 * t.tile_m * t.tile_n * (double)(K / split);
    const double peak = exact ? 4096.0 : 8192.0;   // FLOP per clock per CU
    // under a full MFMA load the part sits at its power cap: measured
    // MFMA work takes ~1.6x its 2.4 GHz cycle count in wall time
    const double compute = flops / (peak * t.rel_rate) * t.blocks_per_cu * 1.6;
    const int64_t stages = ceil_div(K / split / 128, t.steps_per_stage);
    const double copy = (double)stages * 4400.0;
    const double item = (compute > copy ? compute : copy) + 3000.0;
    double total = (double)rounds * item;
    if (split > 1) {
        if (fused_combine(t.tile_m, t.tile_n, split)) {
            // the last split of each tile reads the tile's partials (~12
            // B/clock per CU) after a chain of device-memory round trips
            // (partial stores complete, arrival count, partial loads): ~9000
            // clocks, from runs of one shape with and without the split
            // (128 x 256 x 512, 16 x 64 tiles: 13.3 vs 11.8 us per run)
            total += (double)t.tile_m * t.tile_n * split * 4.0 / 12.0 + 9000.0;
        } else {
            // FP32 partials written and read back, C written, by a second
            // launch: bytes at ~2.5 TB/s (measured), plus the launch
            const double bytes = (double)rows * N * (8.0 * split + 2.0);
            total += bytes / 2.5e12 * 2.4e9 + 5000.0;
        }
    }
    return total;
}

// Flags protocol: the split (a divisor of R) whose K range fits the
// kernel's LDS and whose grid fits one work-group per compute unit, the
// largest such grid; 0 if none.
int ring_split(int64_t kpr, int32_t R, int64_t N, int num_cus)
{
    const int64_t tiles_n = ceil_div(N, mxg::kRingBN);
    int best = 0;
    for (int s = 1; s <= R; ++s) {
        if (R % s != 0 || (int64_t)(R / s) * (kpr / 128) > mxg::kRingMaxSteps)
            continue;
        if (tiles_n * s > num_cus)
            continue;
        if (best == 0 || tiles_n * s > tiles_n * best)
            best = s;
    }
    return best;
}

constexpr int kDefaultSpinLimit = 1 << 19;

int make_plan(mxgemm_seg_plan_t* p, int64_t M, int64_t kpr, int32_t R, int64_t N, int64_t cms,
              int32_t nbuf, int32_t num_cus, const mxgemm_seg_options_t* opts)
{
    int rc = validate(M, kpr, R, N, cms, nbuf);
    if (rc != MXGEMM_OK)
        return rc;
    if (num_cus <= 0)
        return fail(MXGEMM_EINVAL, "num_cus must be positive");
    memset(p, 0, sizeof(*p));
    p->M = M;
    p->kPerRank = kpr;
    p->N = N;
    p->K = (int64_t)R * kpr;
    p->commMSize = cms;
    p->rank_size = R;
    p->buffer_count = nbuf;
    p->chunks = (int32_t)ceil_div(M, cms);   // the last chunk may be short
    p->num_cus = num_cus;
    p->precision = MXGEMM_PRECISION_EXACT;
    if (opts && opts->precision >= 0) {
        if (opts->precision != MXGEMM_PRECISION_EXACT && opts->precision != MXGEMM_PRECISION_NATIVE)
            return fail(MXGEMM_EINVAL, "unknown precision mode %d", opts->precision);
        p->precision = opts->precision;
    }
    const bool exact = p->precision == MXGEMM_PRECISION_EXACT;
    p->a_format = MXGEMM_FMT_E4M3;
    p->b_format = MXGEMM_FMT_E4M3;
    if (opts && opts->a_format >= 0)
        p->a_format = opts->a_format;
    if (opts && opts->b_format >= 0)
        p->b_format = opts->b_format;
    if ((p->a_format != MXGEMM_FMT_E4M3 && p->a_format != MXGEMM_FMT_E5M2) ||
        (p->b_format != MXGEMM_FMT_E4M3 && p->b_format != MXGEMM_FMT_E5M2))
        return fail(MXGEMM_EINVAL, "unknown FP8 format (a %d, b %d)", p->a_format, p->b_format);

    // Window size W (chunks per stage/GEMM launch pair).  W = nbuf / 2
    // lets the staging of window w + 1 overlap the GEMM of window w; W =
    // nbuf gives the GEMM twice the rows (bigger tiles, fuller grid) but the
    // staging of each window then waits for the previous GEMM.  The plan
    // takes the cheaper of the two under the cost model below.
    int w_cand[2] = {nbuf > 1 ? nbuf / 2 : 1, nbuf};
    int n_w = nbuf > 1 ? 2 : 1;
    if (opts && opts->chunks_per_window > 0) {
        if (nbuf % opts->chunks_per_window != 0)
            return fail(MXGEMM_EINVAL, "chunks_per_window %d must divide buffer_count %d",
                        opts->chunks_per_window, nbuf);
        w_cand[0] = opts->chunks_per_window;
        n_w = 1;
    }
    if (opts && opts->tile_cfg >= mxg::num_tile_cfgs())
        return fail(MXGEMM_EINVAL, "tile_cfg %d out of range [0, %d)", opts->tile_cfg,
                    mxg::num_tile_cfgs());
    if (opts && opts->tile_cfg >= 0 && exact && !mxg::tile_cfg(opts->tile_cfg).exact)
        return fail(MXGEMM_EINVAL, "tile_cfg %d (%d x %d) has no exact-mode kernel", opts->tile_cfg,
                    mxg::tile_cfg(opts->tile_cfg).tile_m, mxg::tile_cfg(opts->tile_cfg).tile_n);
    if (opts && opts->tile_cfg >= 0 && !exact && !mxg::tile_cfg(opts->tile_cfg).native)
        return fail(MXGEMM_EINVAL, "tile_cfg %d (%d x %d) has no native-mode kernel", opts->tile_cfg,
                    mxg::tile_cfg(opts->tile_cfg).tile_m, mxg::tile_cfg(opts->tile_cfg).tile_n);

    Choice best = {-1, 1, 1e300, 0};
    int best_w = w_cand[0];
    const int ncfg = mxg::num_tile_cfgs();
    for (int wi = 0; wi < n_w; ++wi) {
        const int W = w_cand[wi];
        const int64_t windows = ceil_div(p->chunks, W);
        const int64_t rows = (int64_t)W * cms;
        // staging one window: read + write of its data and scales at an
        // assumed 4 TB/s, in 2.4 GHz clock cycles
        const double stage = 2.0 * (double)rows * R * kpr * 33.0 / 32.0 / 4.0e12 * 2.4e9;
        const bool overlap = nbuf / W >= 2;
        for (int c = 0; c < ncfg; ++c) {
            if (opts && opts->tile_cfg >= 0 && opts->tile_cfg != c)
                continue;
            if (exact ? !mxg::tile_cfg(c).exact : !mxg::tile_cfg(c).native)
                continue;
            for (int s = 1; s <= R; ++s) {
                if (R % s != 0)
                    continue;
                if (opts && opts->split > 0 && opts->split != s)
                    continue;
                if (c == mxg::kOneShotCfg && (int64_t)(R / s) * (kpr / 128) > mxg::kOneShotSteps)
                    continue;   // a work item's K range must fit the single stage
                if ((int64_t)(R / s) * (kpr / 128) % mxg::tile_cfg(c).k_groups != 0)
                    continue;   // K groups take equal shares of the K-steps
                // Unasked, K groups only with at least 4 K-steps each: fewer
                // do not pay for the groups' final reduction and the unhidden
                // first copy (128 x 256 x 512, one K-step per group: 14.4 us
                // per run against 11.5 us with 16 x 64 tiles)
                if (mxg::tile_cfg(c).k_groups > 1 && !(opts && opts->tile_cfg == c) &&
                    (int64_t)(R / s) * (kpr / 128) < 4LL * mxg::tile_cfg(c).k_groups)
                    continue;
                // Some tiles only when asked for (the one-shot tile: measured
                // against the pipelined 16 x 64 tile, two work-groups per CU,
                // it was slower on every shape it fits -- 64 x 2048 x 7168:
                // 37.4 vs 33.9 us per run; 128 x 256 x 512: 12.2 vs 11.8 us --
                // which this cost model does not predict).
                if (!mxg::tile_cfg(c).automatic && !(opts && opts->tile_cfg == c))
                    continue;
                const double gemm = estimate(mxg::tile_cfg(c), rows, N, p->K, s, num_cus, exact);
                // With two or more slot groups the staging runs on the side
                // stream, and each window pays the ready and credit hand-offs
                // between the streams: ~14 us per window measured on the
                // 8192-cube workload (eight 1024-row windows took 1146 us per
                // run against 1029 us for four 2048-row windows on one
                // stream, the GEMM launches accounting for 1033 and 993 us).
                const double handoff = 14.0e-6 * 2.4e9;
                const double cost = overlap
                    ? (double)windows * ((gemm > stage ? gemm : stage) + handoff) + stage
                    : (double)windows * (gemm + stage);
                // estimates within 0.1% count as a tie, which goes to the
                // plan with more work items: more work-groups in flight hide
                // more latency (128 x 256 x 512: 16 x 64 tiles 11.6 us per
                // run against 12.2 us for 32 x 64 at the same estimate)
                const mxg::TileCfg& tc = mxg::tile_cfg(c);
                const int64_t work = ceil_div(rows, tc.tile_m) * ceil_div(N, tc.tile_n) * s;
                if (cost < best.cost * 0.999 || (cost <= best.cost * 1.001 && work > best.work)) {
                    best.cfg = c;
                    best.split = s;
                    best.cost = cost;
                    best.work = work;
                    best_w = W;
                }
            }
        }
    }
    if (best.cfg < 0)
        return fail(MXGEMM_EINVAL, "no plan satisfies the options (split must divide rank_size; "
                                   "tile_cfg %d needs at most %d K-steps of 128 per split; a tile "
                                   "with K groups needs a multiple of their count)",
                    mxg::kOneShotCfg, mxg::kOneShotSteps);
    const int W = best_w;
    p->chunks_per_window = W;
    p->windows = (int32_t)ceil_div(p->chunks, W);
    p->window_slots = nbuf / W;
    const int64_t rows = (int64_t)W * cms;

    const mxg::TileCfg& t = mxg::tile_cfg(best.cfg);
    p->tile_cfg = best.cfg;
    p->tile_m = t.tile_m;
    p->tile_n = t.tile_n;
    p->split = best.split;
    p->tiles_m = (int32_t)ceil_div(rows, t.tile_m);
    p->tiles_n = (int32_t)ceil_div(N, t.tile_n);
    const int64_t work = (int64_t)p->tiles_m * p->tiles_n * p->split;
    if (work >= (1LL << 31))
        return fail(MXGEMM_EUNSUPPORTED, "too many work items");
    p->work_items = (int32_t)work;
    p->grid = (int32_t)work;
    // zigzag group width: about a square patch of tiles per XCD per round of
    // resident work-groups
    const int64_t resident = (int64_t)num_cus * t.blocks_per_cu;
    const int64_t per_xcd = ceil_div(work < resident ? work : resident, mxg::kNumXcd) / p->split;
    int g = (int)floor(sqrt((double)(per_xcd > 1 ? per_xcd : 1)));
    if (g < 1)
        g = 1;
    if (g > p->tiles_n)
        g = p->tiles_n;
    p->group_n = g;
    p->slot_bytes = (int64_t)R * cms * kpr;
    p->scale_slot_bytes = (int64_t)R * cms * (kpr / 32);
    p->workspace_bytes = p->split > 1 ? (int64_t)p->split * rows * N * 4 : 0;
    p->ring = MXGEMM_RING_EVENTS;
    p->spin_limit = opts && opts->spin_limit >= 0 ? opts->spin_limit : kDefaultSpinLimit;

    // Flags protocol: only when asked for.  Measured against the events
    // protocol it was slower on every shape it fits (64 x 2048 x 7168: 71.8
    // vs 36.7 us per run, stream-issued), its windows being chains of
    // device-memory round trips.
    const int want = opts ? opts->ring : -1;
    if (want != -1 && want != MXGEMM_RING_EVENTS && want != MXGEMM_RING_FLAGS)
        return fail(MXGEMM_EINVAL, "unknown ring protocol %d", want);
    if (want != MXGEMM_RING_FLAGS)
        return MXGEMM_OK;
    const bool forced_tiles = opts && (opts->tile_cfg >= 0 || opts->split > 0);
    int s = !forced_tiles ? ring_split(kpr, R, N, num_cus) : 0;
    // one window per ring fill: each window costs a chain of device-memory
    // hand-overs (64 x 2048 x 7168, 8 ranks, depth 4: 42 us per run with
    // W = 4, 71 us with W = 2, 110 us with W = 1)
    const int Wr = opts && opts->chunks_per_window > 0 ? opts->chunks_per_window : nbuf;
    const int64_t windows_r = ceil_div(p->chunks, Wr);
    const int64_t tiles_m_win = ceil_div((int64_t)Wr * cms, mxg::kRingBM);
    const int64_t tiles_n_r = ceil_div(N, mxg::kRingBN);
    if (s > 0) {
        const int64_t words = mxg::ring_sync_words(nbuf / Wr, s, (int)windows_r, (int)tiles_m_win,
                                                   (int)tiles_n_r);
        const int64_t ws = s > 1 ? (int64_t)s * M * N * 4 : 0;
        if (words > (1 << 20) || ws > (1LL << 32))
            s = 0;
    }
    if (s == 0)
        return fail(MXGEMM_EUNSUPPORTED, "the flags protocol needs no forced tile or split, a "
                    "split whose K range is at most %d K-steps of 128 and at most one "
                    "work-group per compute unit (%d)", mxg::kRingMaxSteps, num_cus);
    p->ring = MXGEMM_RING_FLAGS;
    p->chunks_per_window = Wr;
    p->windows = (int32_t)windows_r;
    p->window_slots = nbuf / Wr;
    p->tile_cfg = -1;
    p->tile_m = mxg::kRingBM;
    p->tile_n = mxg::kRingBN;
    p->split = s;
    p->tiles_m = (int32_t)tiles_m_win;
    p->tiles_n = (int32_t)tiles_n_r;
    p->work_items = (int32_t)(tiles_n_r * s);
    p->grid = p->work_items;
    p->group_n = 1;
    p->workspace_bytes = s > 1 ? (int64_t)s * M * N * 4 : 0;
    return MXGEMM_OK;
}

}  // namespace

struct mxgemm_seg {
    mxgemm_seg_plan_t plan;
    int device;
    const void* checked[5];   // run() buffers last found accessible and large enough
    uint8_t* ring;
    uint8_t* sring;
    float* ws;
    uint32_t* tile_cnt;   // events protocol, fused split-K combine: arrivals per tile
    uint32_t* sync;   // flags protocol: counters, then the error word
    hipStream_t side;
    hipEvent_t start;
    std::vector<hipEvent_t> ready, credit;
    // measurement
    bool profiling;
    bool pending;
    std::vector<hipEvent_t> gemm_ev, stage_ev;
    double gemm_ms, stage_ms;
    int gemm_n, stage_n;
};

namespace {

void release(mxgemm_seg* h)
{
    if (h->side)
        (void)hipStreamSynchronize(h->side);
    for (hipEvent_t e : h->ready)
        (void)hipEventDestroy(e);
    for (hipEvent_t e : h->credit)
        (void)hipEventDestroy(e);
    for (hipEvent_t e : h->gemm_ev)
        (void)hipEventDestroy(e);
    for (hipEvent_t e : h->stage_ev)
        (void)hipEventDestroy(e);
    if (h->start)
        (void)hipEventDestroy(h->start);
    if (h->side)
        (void)hipStreamDestroy(h->side);
    if (h->ring)
        (void)hipFree(h->ring);
    if (h->sring)
        (void)hipFree(h->sring);
    if (h->ws)
        (void)hipFree(h->ws);
    if (h->sync)
        (void)hipFree(h->sync);
    if (h->tile_cnt)
        (void)hipFree(h->tile_cnt);
    delete h;
}

// The run() buffers must be memory the GPU can read: device memory of the
// handle's device, managed memory or pinned host memory.  Pageable host
// memory would fault the kernels, so it is refused before anything is
// enqueued.  Checked whenever the pointers differ from the last ones that
// passed (so a steady loop, and graph capture after an eager run, make no
// extra calls).  Buffer sizes are the caller's contract and are not
// checked: an allocation's range as the runtime reports it need not be all
// of the memory mapped behind a pointer.
int gpu_accessible(const void* p, const char* name, int device)
{
    hipPointerAttribute_t at;
    hipError_t e = hipPointerGetAttributes(&at, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MXGEMM_EINVAL, "%s: no pointer attributes (%s)", name, hipGetErrorString(e));
    }
    if (at.type == hipMemoryTypeDevice) {
        if (at.device != device)
            return fail(MXGEMM_EINVAL, "%s is memory of device %d, not of device %d", name, at.device,
                        device);
        return MXGEMM_OK;
    }
    if (at.type == hipMemoryTypeManaged || at.type == hipMemoryTypeHost)
        return MXGEMM_OK;
    return fail(MXGEMM_EINVAL, "%s is not memory the GPU can access (host memory that is not "
                "pinned?)", name);
}

int check_buffers(mxgemm_seg* h, const void* const (&ptr)[5])
{
    static const char* const names[5] = {"a_seg", "a_scale", "b", "b_scale", "c"};
    bool same = true;
    for (int i = 0; i < 5; ++i)
        same = same && ptr[i] == h->checked[i];
    if (same)
        return MXGEMM_OK;
    for (int i = 0; i < 5; ++i) {
        int rc = gpu_accessible(ptr[i], names[i], h->device);
        if (rc != MXGEMM_OK)
            return rc;
    }
    for (int i = 0; i < 5; ++i)
        h->checked[i] = ptr[i];
    return MXGEMM_OK;
}

int harvest(mxgemm_seg* h)
{
    if (!h->pending)
        return MXGEMM_OK;
    h->pending = false;
    if (h->plan.ring == MXGEMM_RING_FLAGS) {
        HIP_TRY(hipEventSynchronize(h->gemm_ev[1]));
        float ms = 0.f;
        HIP_TRY(hipEventElapsedTime(&ms, h->gemm_ev[0], h->gemm_ev[1]));
        h->gemm_ms += ms;
        h->gemm_n += 1;
        return MXGEMM_OK;
    }
    const int nw = h->plan.windows;
    HIP_TRY(hipEventSynchronize(h->gemm_ev[2 * nw - 1]));
    HIP_TRY(hipEventSynchronize(h->stage_ev[2 * nw - 1]));
    for (int w = 0; w < nw; ++w) {
        float ms = 0.f;
        HIP_TRY(hipEventElapsedTime(&ms, h->gemm_ev[2 * w], h->gemm_ev[2 * w + 1]));
        h->gemm_ms += ms;
        HIP_TRY(hipEventElapsedTime(&ms, h->stage_ev[2 * w], h->stage_ev[2 * w + 1]));
        h->stage_ms += ms;
    }
    h->gemm_n += nw;
    h->stage_n += nw;
    return MXGEMM_OK;
}

// Events protocol: for each window, the staging kernel, the ready
// hand-over, the GEMM (and a split-K reduce), the credit hand-over; the
// buffers are the handle's (or, for the static-scratch entry, the scratch
// array's).
int enqueue_events(mxgemm_seg* h, const void* a_seg, const void* a_scale, const void* b,
                   const void* b_scale, void* c, hipStream_t st)
{
    const mxgemm_seg_plan_t& P = h->plan;
    // With one slot group the staging of a window waits for the GEMM of the
    // previous one anyway: both run on `stream`, whose order is then the
    // ready/credit order (no cross-stream hand-offs, each of which costs
    // tens of microseconds between these kernels).  Otherwise the staging
    // runs on the side stream, forked from `stream`, so that it can run
    // ahead of the GEMMs.
    const bool one_stream = P.window_slots == 1;
    hipStream_t producer = one_stream ? st : h->side;
    if (!one_stream) {
        HIP_TRY(hipEventRecord(h->start, st));
        HIP_TRY(hipStreamWaitEvent(h->side, h->start, 0));
    }

    for (int w = 0; w < P.windows; ++w) {
        const int chunk0 = w * P.chunks_per_window;
        const int left = P.chunks - chunk0;
        const int nch = left < P.chunks_per_window ? left : P.chunks_per_window;
        const int g = w % P.window_slots;

        // producer: refill slot group g once the GEMM that last read it is done
        if (!one_stream && w >= P.window_slots)
            HIP_TRY(hipStreamWaitEvent(h->side, h->credit[g], 0));
        mxg::StageArgs sa;
        sa.a_seg = (const uint8_t*)a_seg;
        sa.sa_seg = (const uint8_t*)a_scale;
        sa.ring = h->ring;
        sa.sring = h->sring;
        sa.M = P.M;
        sa.kpr = P.kPerRank;
        sa.cms = P.commMSize;
        sa.slot_bytes = P.slot_bytes;
        sa.scale_slot_bytes = P.scale_slot_bytes;
        sa.R = P.rank_size;
        sa.chunk0 = chunk0;
        sa.nch = nch;
        sa.nbuf = P.buffer_count;
        if (h->profiling)
            HIP_TRY(hipEventRecord(h->stage_ev[2 * w], producer));
        HIP_TRY(mxg::launch_stage(sa, producer));
        if (h->profiling)
            HIP_TRY(hipEventRecord(h->stage_ev[2 * w + 1], producer));
        if (!one_stream) {
            HIP_TRY(hipEventRecord(h->ready[g], h->side));
            // consumer: GEMM over the window once its chunks have landed
            HIP_TRY(hipStreamWaitEvent(st, h->ready[g], 0));
        }
        // rows of the window: whole chunks, except that the last chunk of
        // the problem holds only the rows left
        const int64_t rows_left = P.M - (int64_t)chunk0 * P.commMSize;
        const int64_t rows = (int64_t)nch * P.commMSize < rows_left ? (int64_t)nch * P.commMSize
                                                                       : rows_left;
        mxg::GemmArgs ga;
        ga.a = h->ring + (int64_t)g * P.chunks_per_window * P.slot_bytes;
        ga.as = h->sring + (int64_t)g * P.chunks_per_window * P.scale_slot_bytes;
        ga.a_slot_stride = P.slot_bytes;
        ga.as_slot_stride = P.scale_slot_bytes;
        ga.b = (const uint8_t*)b;
        ga.bs = (const uint8_t*)b_scale;
        ga.c = (uint16_t*)c + (int64_t)chunk0 * P.commMSize * P.N;
        ga.ws = h->ws;
        ga.tile_cnt = h->tile_cnt;
        ga.fused = fused_combine(P.tile_m, P.tile_n, P.split) ? 1 : 0;
        ga.rows = (int)rows;
        ga.N = (int)P.N;
        ga.K = (int)P.K;
        ga.kpr = (int)P.kPerRank;
        ga.cms = (int)P.commMSize;
        ga.tiles_m = (int)ceil_div(rows, P.tile_m);
        ga.tiles_n = P.tiles_n;
        ga.split = P.split;
        ga.segs_per_split = P.rank_size / P.split;
        ga.group_n = P.group_n;
        ga.total_work = ga.tiles_m * ga.tiles_n * ga.split;
        ga.c_vec4 = ((uintptr_t)ga.c % 8 == 0) && (P.N % 4 == 0);
        if (h->profiling)
            HIP_TRY(hipEventRecord(h->gemm_ev[2 * w], st));
        HIP_TRY(mxg::launch_gemm(P.tile_cfg, P.precision == MXGEMM_PRECISION_EXACT, P.a_format,
                                 P.b_format, ga, st));
        if (h->profiling)
            HIP_TRY(hipEventRecord(h->gemm_ev[2 * w + 1], st));
        if (P.split > 1 && !ga.fused) {
            mxg::ReduceArgs ra;
            ra.ws = h->ws;
            ra.c = ga.c;
            ra.rows = ga.rows;
            ra.N = ga.N;
            ra.split = P.split;
            ra.c_vec4 = ga.c_vec4;
            HIP_TRY(mxg::launch_reduce(ra, st));
        }
        if (!one_stream)
            HIP_TRY(hipEventRecord(h->credit[g], st));
    }
    if (h->profiling)
        h->pending = true;
    return MXGEMM_OK;
}

// ---- static scratch: the entry point that allocates nothing -----------
//
// mxgemm_seg_run_static keeps the ring, the split-K workspace and the
// per-tile arrival counts in this file-scope array instead of memory that
// create() allocates.  In host code `scratch` is only a stand-in for the
// symbol; its device address on each GPU comes from hipGetSymbolAddress,
// taken once per device (with that device current) and kept in
// g_static[device].ptr, which is what every launch receives.
constexpr int64_t kStaticScratchBytes = 32LL << 20;
constexpr int kMaxStaticDevices = 64;

struct StaticDevice {
    bool ready;
    uint8_t* ptr;              // device address of `scratch` on this device
    int num_cus;
    const void* checked[5];    // run buffers last found accessible
};

std::mutex g_static_mu;
StaticDevice g_static[kMaxStaticDevices];

}  // namespace

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

// Per-device set-up, once: the device must be a gfx950, and the scratch
// array's address on it is looked up (never the symbol's host stand-in).
int static_device(int dev, StaticDevice** out)
{
    std::lock_guard<std::mutex> lock(g_static_mu);
    if (dev < 0 || dev >= kMaxStaticDevices)
        return fail(MXGEMM_EUNSUPPORTED, "device index %d out of range", dev);
    StaticDevice& sd = g_static[dev];
    if (!sd.ready) {
        hipDeviceProp_t prop;
        HIP_TRY(hipGetDeviceProperties(&prop, dev));
        if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
            return fail(MXGEMM_EUNSUPPORTED, "device %d is %s; this library is built for gfx950",
                        dev, prop.gcnArchName);
        void* ptr = nullptr;
        HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
        if (ptr == nullptr)
            return fail(MXGEMM_EHIP, "no device address for the static scratch array");
        sd.ptr = static_cast<uint8_t*>(ptr);
        sd.num_cus = prop.multiProcessorCount;
        sd.ready = true;
    }
    *out = &sd;
    return MXGEMM_OK;
}

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

}  // namespace

extern "C" {

const char* mxgemm_seg_last_error(void) { return g_err.c_str(); }

int mxgemm_seg_plan(mxgemm_seg_plan_t* out, int64_t M, int64_t kPerRank, int32_t rank_size,
                    int64_t N, int64_t commMSize, int32_t buffer_count, int32_t num_cus,
                    const mxgemm_seg_options_t* opts)
{
    if (!out)
        return fail(MXGEMM_EINVAL, "out is NULL");
    mxgemm_seg_plan_t p;
    int rc = make_plan(&p, M, kPerRank, rank_size, N, commMSize, buffer_count, num_cus, opts);
    if (rc == MXGEMM_OK)
        *out = p;
    return rc;
}

int mxgemm_seg_decode(const mxgemm_seg_plan_t* plan, int64_t rows, int32_t w, int32_t block,
                      int32_t* tile_m_idx, int32_t* tile_n_idx, int32_t* split_idx,
                      int32_t* first_work)
{
    if (!plan || rows <= 0 || rows > (int64_t)plan->chunks_per_window * plan->commMSize)
        return fail(MXGEMM_EINVAL, "bad plan or rows");
    if (plan->ring != MXGEMM_RING_EVENTS)
        return fail(MXGEMM_EINVAL, "work IDs are decoded for the events protocol only");
    const int tiles_m = (int)ceil_div(rows, plan->tile_m);
    const int total = tiles_m * plan->tiles_n * plan->split;
    const int grid = total;   // one work-group per work item
    if (w < 0 || w >= total || block < 0 || block >= grid)
        return fail(MXGEMM_EINVAL, "work item or block out of range");
    const mxg::TileCoord c = mxg::decode_work(w, tiles_m, plan->tiles_n, plan->split, plan->group_n);
    if (tile_m_idx)
        *tile_m_idx = c.tm;
    if (tile_n_idx)
        *tile_n_idx = c.tn;
    if (split_idx)
        *split_idx = c.ks;
    if (first_work)
        *first_work = mxg::remap_block(block, grid);
    return MXGEMM_OK;
}

int mxgemm_seg_create_ex(mxgemm_seg_t* out, int64_t M, int64_t kPerRank, int32_t rank_size,
                         int64_t N, int64_t commMSize, int32_t buffer_count,
                         const mxgemm_seg_options_t* opts)
{
    if (!out)
        return fail(MXGEMM_EINVAL, "out is NULL");
    int rc = validate(M, kPerRank, rank_size, N, commMSize, buffer_count);
    if (rc != MXGEMM_OK)
        return rc;
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    hipDeviceProp_t prop;
    HIP_TRY(hipGetDeviceProperties(&prop, dev));
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(MXGEMM_EUNSUPPORTED, "device %d is %s; this library is built for gfx950",
                    dev, prop.gcnArchName);
    mxgemm_seg_plan_t plan;
    rc = make_plan(&plan, M, kPerRank, rank_size, N, commMSize, buffer_count,
                   prop.multiProcessorCount, opts);
    if (rc != MXGEMM_OK)
        return rc;

    mxgemm_seg* h = new mxgemm_seg();
    h->plan = plan;
    h->device = dev;
    auto oom = [&](const char* what, size_t bytes) {
        // the failed hipMalloc also set the thread's last HIP error; clear
        // it, or the next launch check (hipGetLastError) would report it
        (void)hipGetLastError();
        release(h);
        return fail(MXGEMM_ENOMEM, "allocating %s (%zu bytes) failed", what, bytes);
    };
    const size_t ring_bytes = (size_t)plan.buffer_count * plan.slot_bytes;
    const size_t sring_bytes = (size_t)plan.buffer_count * plan.scale_slot_bytes;
    if (hipMalloc((void**)&h->ring, ring_bytes) != hipSuccess)
        return oom("staging ring", ring_bytes);
    if (hipMalloc((void**)&h->sring, sring_bytes) != hipSuccess)
        return oom("staging scale ring", sring_bytes);
    if (plan.workspace_bytes > 0 && hipMalloc((void**)&h->ws, plan.workspace_bytes) != hipSuccess)
        return oom("split-K workspace", plan.workspace_bytes);
    if (plan.ring == MXGEMM_RING_EVENTS && fused_combine(plan.tile_m, plan.tile_n, plan.split)) {
        // arrival counts start at zero; every launch leaves them at zero
        const size_t bytes = 4 * (size_t)plan.tiles_m * plan.tiles_n;
        if (hipMalloc((void**)&h->tile_cnt, bytes) != hipSuccess)
            return oom("split-K tile counters", bytes);
        if (hipMemset(h->tile_cnt, 0, bytes) != hipSuccess) {
            (void)hipGetLastError();
            release(h);
            return fail(MXGEMM_EHIP, "clearing the split-K tile counters failed");
        }
    }
    if (plan.ring == MXGEMM_RING_FLAGS) {
        // counters start at zero; each run leaves them at zero
        const size_t bytes = 4 * (size_t)(mxg::ring_sync_words(plan.window_slots, plan.split,
                                                               plan.windows, plan.tiles_m,
                                                               plan.tiles_n) + 1);
        if (hipMalloc((void**)&h->sync, bytes) != hipSuccess)
            return oom("ring counters", bytes);
        if (hipMemset(h->sync, 0, bytes) != hipSuccess) {
            (void)hipGetLastError();
            release(h);
            return fail(MXGEMM_EHIP, "clearing the ring counters failed");
        }
    }
    hipError_t e = hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking);
    if (e == hipSuccess)
        e = hipEventCreateWithFlags(&h->start, hipEventDisableTiming);
    h->ready.assign(plan.window_slots, nullptr);
    h->credit.assign(plan.window_slots, nullptr);
    for (int i = 0; e == hipSuccess && i < plan.window_slots; ++i) {
        e = hipEventCreateWithFlags(&h->ready[i], hipEventDisableTiming);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&h->credit[i], hipEventDisableTiming);
    }
    if (e == hipSuccess)
        e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        (void)hipGetLastError();
        release(h);
        return fail(MXGEMM_EHIP, "handle setup failed: %s", hipGetErrorString(e));
    }
    *out = h;
    return MXGEMM_OK;
}

int mxgemm_seg_create(mxgemm_seg_t* out, int64_t M, int64_t kPerRank, int32_t rank_size,
                      int64_t N, int64_t commMSize, int32_t buffer_count)
{
    return mxgemm_seg_create_ex(out, M, kPerRank, rank_size, N, commMSize, buffer_count, nullptr);
}

int mxgemm_seg_get_plan(mxgemm_seg_t h, mxgemm_seg_plan_t* out)
{
    if (!h || !out)
        return fail(MXGEMM_EINVAL, "NULL handle or out");
    *out = h->plan;
    return MXGEMM_OK;
}

int mxgemm_seg_run(mxgemm_seg_t h, const void* a_seg, const void* a_scale, const void* b,
                   const void* b_scale, void* c, void* stream)
{
    if (!h)
        return fail(MXGEMM_EINVAL, "NULL handle");
    if (!a_seg || !a_scale || !b || !b_scale || !c)
        return fail(MXGEMM_EINVAL, "NULL data pointer");
    if (((uintptr_t)a_seg | (uintptr_t)b) & 15u)
        return fail(MXGEMM_EINVAL, "a_seg and b must be 16-byte aligned");
    if (((uintptr_t)a_scale | (uintptr_t)b_scale) & 3u)
        return fail(MXGEMM_EINVAL, "a_scale and b_scale must be 4-byte aligned");
    if ((uintptr_t)c & 1u)
        return fail(MXGEMM_EINVAL, "c must be 2-byte aligned");
    const mxgemm_seg_plan_t& P = h->plan;
    hipStream_t st = (hipStream_t)stream;
    {
        const void* const ptr[5] = {a_seg, a_scale, b, b_scale, c};
        int rc = check_buffers(h, ptr);
        if (rc != MXGEMM_OK)
            return rc;
    }

    if (h->profiling) {
        int rc = harvest(h);
        if (rc != MXGEMM_OK)
            return rc;
    }

    if (P.ring == MXGEMM_RING_FLAGS) {
        mxg::RingArgs ra;
        ra.a_seg = (const uint8_t*)a_seg;
        ra.sa_seg = (const uint8_t*)a_scale;
        ra.ring = h->ring;
        ra.sring = h->sring;
        ra.b = (const uint8_t*)b;
        ra.bs = (const uint8_t*)b_scale;
        ra.c = (uint16_t*)c;
        ra.ws = h->ws;
        ra.sync = h->sync;
        ra.err = h->sync + mxg::ring_sync_words(P.window_slots, P.split, P.windows, P.tiles_m,
                                                P.tiles_n);
        ra.M = P.M;
        ra.kpr = P.kPerRank;
        ra.cms = P.commMSize;
        ra.slot_bytes = P.slot_bytes;
        ra.scale_slot_bytes = P.scale_slot_bytes;
        ra.R = P.rank_size;
        ra.N = (int)P.N;
        ra.K = (int)P.K;
        ra.nbuf = P.buffer_count;
        ra.chunks = P.chunks;
        ra.W = P.chunks_per_window;
        ra.windows = P.windows;
        ra.window_slots = P.window_slots;
        ra.tiles_n = P.tiles_n;
        ra.split = P.split;
        ra.segs_per_split = P.rank_size / P.split;
        ra.tiles_m_win = P.tiles_m;
        ra.c_vec4 = ((uintptr_t)c % 8 == 0) && (P.N % 4 == 0);
        ra.spin_limit = P.spin_limit;
        if (h->profiling)
            HIP_TRY(hipEventRecord(h->gemm_ev[0], st));
        HIP_TRY(mxg::launch_ring(ra, P.a_format, P.b_format, P.precision == MXGEMM_PRECISION_EXACT, st));
        if (h->profiling) {
            HIP_TRY(hipEventRecord(h->gemm_ev[1], st));
            h->pending = true;
        }
        return MXGEMM_OK;
    }

    return enqueue_events(h, a_seg, a_scale, b, b_scale, c, st);
}

int mxgemm_seg_run_static(int64_t M, int64_t kPerRank, int32_t rank_size, int64_t N,
                          int64_t commMSize, int32_t buffer_count, const mxgemm_seg_options_t* opts,
                          const void* a_seg, const void* a_scale, const void* b,
                          const void* b_scale, void* c, void* stream)
{
    mxgemm_seg_options_t o;
    if (opts) {
        o = *opts;
        if (o.ring != -1 && o.ring != MXGEMM_RING_EVENTS)
            return fail(MXGEMM_EUNSUPPORTED, "the static-scratch entry runs the events protocol only");
        if (o.chunks_per_window != -1 && o.chunks_per_window != buffer_count)
            return fail(MXGEMM_EINVAL, "the static-scratch entry uses one window per ring fill "
                        "(chunks_per_window must be -1 or buffer_count)");
    } else {
        memset(&o, 0xFF, sizeof(o));           // every knob -1: automatic
    }
    // one slot group: staging and GEMM in order on `stream`, no side stream
    // or events (which create() would have to allocate)
    o.chunks_per_window = buffer_count;
    o.ring = MXGEMM_RING_EVENTS;
    int rc = validate(M, kPerRank, rank_size, N, commMSize, buffer_count);
    if (rc != MXGEMM_OK)
        return rc;
    if (!a_seg || !a_scale || !b || !b_scale || !c)
        return fail(MXGEMM_EINVAL, "NULL data pointer");
    if (((uintptr_t)a_seg | (uintptr_t)b) & 15u)
        return fail(MXGEMM_EINVAL, "a_seg and b must be 16-byte aligned");
    if (((uintptr_t)a_scale | (uintptr_t)b_scale) & 3u)
        return fail(MXGEMM_EINVAL, "a_scale and b_scale must be 4-byte aligned");
    if ((uintptr_t)c & 1u)
        return fail(MXGEMM_EINVAL, "c must be 2-byte aligned");
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    StaticDevice* sd = nullptr;
    rc = static_device(dev, &sd);
    if (rc != MXGEMM_OK)
        return rc;

    mxgemm_seg h{};                            // lives for this call; owns nothing
    rc = make_plan(&h.plan, M, kPerRank, rank_size, N, commMSize, buffer_count, sd->num_cus, &o);
    if (rc != MXGEMM_OK)
        return rc;
    const mxgemm_seg_plan_t& P = h.plan;
    const bool fused = fused_combine(P.tile_m, P.tile_n, P.split);
    const int64_t ring_bytes = align256((int64_t)P.buffer_count * P.slot_bytes);
    const int64_t sring_bytes = align256((int64_t)P.buffer_count * P.scale_slot_bytes);
    const int64_t ws_bytes = align256(P.workspace_bytes);
    const int64_t cnt_words = fused ? (int64_t)P.tiles_m * P.tiles_n : 0;
    const int64_t need = ring_bytes + sring_bytes + ws_bytes + align256(4 * cnt_words);
    if (need > kStaticScratchBytes)
        return fail(MXGEMM_EUNSUPPORTED, "this problem needs %lld bytes of ring and workspace, "
                    "more than the %lld-byte static scratch; use mxgemm_seg_create",
                    (long long)need, (long long)kStaticScratchBytes);

    {
        const void* const ptr[5] = {a_seg, a_scale, b, b_scale, c};
        static const char* const names[5] = {"a_seg", "a_scale", "b", "b_scale", "c"};
        std::lock_guard<std::mutex> lock(g_static_mu);
        bool same = true;
        for (int i = 0; i < 5; ++i)
            same = same && ptr[i] == sd->checked[i];
        if (!same) {
            for (int i = 0; i < 5; ++i) {
                rc = gpu_accessible(ptr[i], names[i], dev);
                if (rc != MXGEMM_OK)
                    return rc;
            }
            for (int i = 0; i < 5; ++i)
                sd->checked[i] = ptr[i];
        }
    }

    h.device = dev;
    h.ring = sd->ptr;
    h.sring = sd->ptr + ring_bytes;
    h.ws = P.workspace_bytes > 0 ? reinterpret_cast<float*>(sd->ptr + ring_bytes + sring_bytes) : nullptr;
    h.tile_cnt = fused ? reinterpret_cast<uint32_t*>(sd->ptr + ring_bytes + sring_bytes + ws_bytes)
                       : nullptr;
    hipStream_t st = (hipStream_t)stream;
    // the arrival counts must start at zero; the array keeps whatever the
    // last call left in this region (ring bytes of a bigger problem, say)
    if (fused)
        HIP_TRY(mxg::launch_fill_u32(h.tile_cnt, cnt_words, 0u, st));
    return enqueue_events(&h, a_seg, a_scale, b, b_scale, c, st);
}

int mxgemm_seg_status(mxgemm_seg_t h)
{
    if (!h)
        return fail(MXGEMM_EINVAL, "NULL handle");
    if (h->plan.ring != MXGEMM_RING_FLAGS)
        return MXGEMM_OK;
    const mxgemm_seg_plan_t& P = h->plan;
    uint32_t* err = h->sync + mxg::ring_sync_words(P.window_slots, P.split, P.windows, P.tiles_m,
                                                   P.tiles_n);
    uint32_t v = 0;
    HIP_TRY(hipDeviceSynchronize());
    HIP_TRY(hipMemcpy(&v, err, 4, hipMemcpyDeviceToHost));
    if (v != 0) {
        HIP_TRY(hipMemset(err, 0, 4));
        HIP_TRY(hipDeviceSynchronize());
        return fail(MXGEMM_ETIMEOUT, "a device wait of the flags protocol gave up");
    }
    return MXGEMM_OK;
}

int mxgemm_seg_destroy(mxgemm_seg_t h)
{
    if (!h)
        return MXGEMM_OK;
    hipError_t e = hipSuccess;
    if (h->side)
        e = hipStreamSynchronize(h->side);
    if (e == hipSuccess)
        e = hipDeviceSynchronize();
    release(h);
    if (e != hipSuccess)
        return fail(MXGEMM_EHIP, "destroy: %s", hipGetErrorString(e));
    return MXGEMM_OK;
}

int mxgemm_seg_set_profiling(mxgemm_seg_t h, int32_t enable)
{
    if (!h)
        return fail(MXGEMM_EINVAL, "NULL handle");
    if (enable && h->gemm_ev.empty()) {
        const int n = 2 * h->plan.windows;
        h->gemm_ev.assign(n, nullptr);
        h->stage_ev.assign(n, nullptr);
        for (int i = 0; i < n; ++i) {
            HIP_TRY(hipEventCreate(&h->gemm_ev[i]));
            HIP_TRY(hipEventCreate(&h->stage_ev[i]));
        }
    }
    if (!enable) {
        int rc = harvest(h);
        if (rc != MXGEMM_OK)
            return rc;
    }
    h->profiling = enable != 0;
    return MXGEMM_OK;
}

int mxgemm_seg_kernel_times(mxgemm_seg_t h, double* gemm_ms, int32_t* gemm_launches,
                            double* stage_ms, int32_t* stage_launches)
{
    if (!h)
        return fail(MXGEMM_EINVAL, "NULL handle");
    int rc = harvest(h);
    if (rc != MXGEMM_OK)
        return rc;
    if (gemm_ms)
        *gemm_ms = h->gemm_ms;
    if (gemm_launches)
        *gemm_launches = h->gemm_n;
    if (stage_ms)
        *stage_ms = h->stage_ms;
    if (stage_launches)
        *stage_launches = h->stage_n;
    h->gemm_ms = h->stage_ms = 0.0;
    h->gemm_n = h->stage_n = 0;
    return MXGEMM_OK;
}

int mxgemm_quantize_mxfp8(const float* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                          int64_t ld_q, uint8_t* s, int64_t ld_s, void* stream)
{
    return mxgemm_quantize_mx(x, rows, cols, ld_x, q, ld_q, s, ld_s, MXGEMM_FMT_E4M3, stream);
}

int mxgemm_quantize_mx(const float* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                       int64_t ld_q, uint8_t* s, int64_t ld_s, int32_t format, void* stream)
{
    if (format != MXGEMM_FMT_E4M3 && format != MXGEMM_FMT_E5M2)
        return fail(MXGEMM_EINVAL, "unknown FP8 format %d", format);
    if (!x || !q || !s)
        return fail(MXGEMM_EINVAL, "NULL pointer");
    if (rows < 0 || cols < 0 || cols % 32 != 0)
        return fail(MXGEMM_EINVAL, "cols must be a non-negative multiple of 32");
    if (ld_x < cols || ld_q < cols || ld_s < cols / 32)
        return fail(MXGEMM_EINVAL, "leading dimensions smaller than the row length");
    if (ld_x % 4 != 0 || ld_q % 4 != 0 || ((uintptr_t)x & 15u) || ((uintptr_t)q & 3u))
        return fail(MXGEMM_EINVAL, "x must be 16-byte aligned with ld_x % 4 == 0; q 4-byte "
                    "aligned with ld_q % 4 == 0");
    if (rows > 0 && cols > 0) {
        int dev = 0;
        HIP_TRY(hipGetDevice(&dev));
        int rc = gpu_accessible(x, "x", dev);
        if (rc == MXGEMM_OK)
            rc = gpu_accessible(q, "q", dev);
        if (rc == MXGEMM_OK)
            rc = gpu_accessible(s, "s", dev);
        if (rc != MXGEMM_OK)
            return rc;
    }
    mxg::QuantArgs a;
    a.x = x;
    a.q = q;
    a.s = s;
    a.rows = rows;
    a.cols = cols;
    a.ld_x = ld_x;
    a.ld_q = ld_q;
    a.ld_s = ld_s;
    a.fmt = format;
    HIP_TRY(mxg::launch_quantize(a, (hipStream_t)stream));
    return MXGEMM_OK;
}

}  // extern "C"
