// soft_topk.hip -- host orchestration and the C ABI (include/soft_topk.h).
//
// Route of one forward call (aiqbench.com abstract of Fast LapSum;
// gist.science summary, section 2.2, "Probabilistic Bracketing" steps 1-4):
//   sample -> select bracket -> pass-1 (tails + band) -> the band's
//   partition refinement (one work-group, or a chain of step kernels),
//   whose steps certify the bracket -> emit p with its fp64 mass partials
//   (folded and checked on request) -> one status read-back.
// Vectors of at most 8192 scores take one kernel instead (a sort and the
// full-sort solve in one work-group).  A rejected bracket widens on the
// failing side (the other end becomes the rejected end, which is then a
// proven bound) and reruns pass-1; an overfull band is refined over every
// score; a refinement that does not end sorts the band (the sorted routes,
// also forced by the parameters); an overfull sorted band splits off a tied
// cluster; a failed mass check or exhausted widenings take the full device
// radix sort, whose solve needs no bracket.  The host only chooses among
// these routes; every step of the arithmetic runs in the kernels.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "soft_topk.h"
#include "stk_common.hpp"
#include "stk_layout.hpp"

namespace stk {

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

thread_local int g_last_hip = 0;

int hip_fail(hipError_t e)
{
    g_last_hip = (int)e;
    return SOFT_TOPK_EHIP;
}

#define STK_HIP(expr)                         \
    do {                                      \
        const hipError_t e_ = (expr);         \
        if (e_ != hipSuccess)                 \
            return hip_fail(e_);              \
    } while (0)

int32_t grid_for(int64_t n, int tile_scores, int cap)
{
    const int64_t g = (n + tile_scores - 1) / tile_scores;
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>(g, cap));
}

// Pass 1 keeps about kPass1TilesPerGroup tiles per work-group (its per-group
// cost -- the status read, the band flush, the partial -- is latency), with
// at least one work-group per CU when there are that many tiles.
int32_t pass1_blocks(int64_t n)
{
    const int64_t tiles = (n + kPass1TileScores - 1) / kPass1TileScores;
    const int64_t spread = std::min<int64_t>(tiles, kCUs);
    const int64_t g = std::max<int64_t>(spread, tiles / kPass1TilesPerGroup);
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>(g, kGridPass1));
}
int32_t emit_blocks(int64_t n)
{
    return grid_for(n, 4 * kStreamThreads * (n >= kStreamLargeMin ? kEmitBatchLarge : kEmitBatchSmall), kGridEmit);
}
int32_t vjp_tile(int64_t n) { return 4 * kStreamThreads * (n >= kStreamLargeMin ? kVjpBatchLarge : kVjpBatchSmall); }
int32_t vjp_grid_cap(int64_t n) { return n >= kStreamLargeMin ? kGridVjpLarge : kGridVjpSmall; }
int32_t vjp_reduce_blocks(int64_t n) { return grid_for(n, vjp_tile(n), vjp_grid_cap(n)); }
// grid of a segment VJP kernel: at most one work-group per large VJP tile
int32_t seg_grid(int64_t n, int32_t cap) { return grid_for(n, 4 * kStreamThreads * kVjpBatchLarge, cap); }
// reduction partials to provide for: either VJP route
int32_t vjp_partial_blocks(int64_t n)
{
    return n >= kSegMinN ? std::max(vjp_reduce_blocks(n), seg_grid(n, kGridVjpSegReduce)) : vjp_reduce_blocks(n);
}
int32_t vjp_apply_blocks(int64_t n) { return grid_for(n, vjp_tile(n), vjp_grid_cap(n)); }

int64_t default_cap(int64_t n)
{
    int64_t c = n / 4;
    c = std::max<int64_t>(c, 1 << 16);
    c = std::min<int64_t>(c, 1 << 22);
    return std::min<int64_t>(c, n);
}

void fill_defaults(soft_topk_params* p)
{
    p->seed = 0x5eedull;
    p->samples = 65536;
    p->z = 5.0;
    p->band_capacity = 0;
    p->max_widen = 2;
    p->force_path = 0;
    p->mass_tolerance = 0.0;
    p->verify_mass = 0;
    p->band_route = 0;
}

bool params_ok(const soft_topk_params& p)
{
    if (p.samples < 1024 || p.samples > 262144)
        return false;
    if (!(p.z > 0.0) || !isfinite(p.z) || p.z > 30.0)
        return false;
    if (p.band_capacity < 0 || p.max_widen < 0 || p.max_widen > 16)
        return false;
    if (p.force_path != 0 && p.force_path != SOFT_TOPK_PATH_BRACKET && p.force_path != SOFT_TOPK_PATH_FULLSORT)
        return false;
    if (!isfinite(p.mass_tolerance))
        return false;
    if (p.verify_mass != 0 && p.verify_mass != 1)
        return false;
    if (p.band_route != 0 && p.band_route != SOFT_TOPK_BAND_DIRECT && p.band_route != SOFT_TOPK_BAND_BUCKETS &&
        p.band_route != SOFT_TOPK_BAND_REFINE && p.band_route != SOFT_TOPK_BAND_REFINE_STEPS)
        return false;
    return true;
}

// ---- binomial rank arithmetic --------------------------------------------
double log_pmf(int64_t m, double q, int64_t i)
{
    return lgamma((double)m + 1.0) - lgamma((double)i + 1.0) - lgamma((double)(m - i) + 1.0) +
           (double)i * log(q) + (double)(m - i) * log1p(-q);
}

// P(X <= r), X ~ Binomial(m, q), for r below the mean: summed from r
// downward with the ratio pmf(i-1)/pmf(i) = i (1-q) / ((m-i+1) q).
double cdf_le(int64_t m, double q, int64_t r)
{
    if (r < 0)
        return 0.0;
    if (r >= m)
        return 1.0;
    double t = exp(log_pmf(m, q, r));
    double s = t;
    const double ratio_q = (1.0 - q) / q;
    for (int64_t i = r; i >= 1; --i) {
        t *= (double)i / (double)(m - i + 1) * ratio_q;
        s += t;
        if ((double)i < (double)m * q && t < 1e-20 * s)
            break;
        if (s > 1.0)
            return 1.0;
    }
    return std::min(s, 1.0);
}

// P(X >= r) for r above the mean: summed upward with
// pmf(i+1)/pmf(i) = (m-i) q / ((i+1) (1-q)).
double sf_ge(int64_t m, double q, int64_t r)
{
    if (r <= 0)
        return 1.0;
    if (r > m)
        return 0.0;
    double t = exp(log_pmf(m, q, r));
    double s = t;
    const double ratio_q = q / (1.0 - q);
    for (int64_t i = r; i < m; ++i) {
        t *= (double)(m - i) / (double)(i + 1) * ratio_q;
        s += t;
        if ((double)i > (double)m * q && t < 1e-20 * s)
            break;
        if (s > 1.0)
            return 1.0;
    }
    return std::min(s, 1.0);
}

// Lower rank: largest r >= 1 with P(X <= r-1) <= delta, else 0 (= -inf).
int64_t lower_rank_exact(int64_t m, double q, double z)
{
    const double delta = 0.5 * erfc(z / sqrt(2.0));
    const double sd = sqrt((double)m * q * (1.0 - q));
    int64_t r = (int64_t)floor((double)m * q - z * sd);
    r = std::max<int64_t>(0, std::min<int64_t>(r, m));
    while (r >= 1 && cdf_le(m, q, r - 1) > delta)
        --r;
    while (r + 1 <= m && cdf_le(m, q, r) <= delta)
        ++r;
    if (r >= 1 && cdf_le(m, q, r - 1) > delta)
        r = 0;
    return r;
}

// Upper rank: smallest r <= m with P(X >= r) <= delta, else m + 1 (= +inf).
int64_t upper_rank_exact(int64_t m, double q, double z)
{
    const double delta = 0.5 * erfc(z / sqrt(2.0));
    const double sd = sqrt((double)m * q * (1.0 - q));
    int64_t r = (int64_t)ceil((double)m * q + z * sd) + 1;
    r = std::max<int64_t>(1, std::min<int64_t>(r, m + 1));
    while (r <= m && sf_ge(m, q, r) > delta)
        ++r;
    while (r - 1 >= 1 && sf_ge(m, q, r - 1) <= delta)
        --r;
    return r;
}

// The ranks depend only on (m, q, z); a small per-thread cache keeps the
// tail sums off the per-call path.
struct RankMemo {
    int64_t m;
    double q, z;
    int64_t rl, rr;
    bool used;
};
thread_local RankMemo g_rank_memo[8];
thread_local int g_rank_next = 0;

void bracket_ranks(int64_t m, double q, double z, int64_t* rl, int64_t* rr)
{
    for (const RankMemo& e : g_rank_memo) {
        if (e.used && e.m == m && e.q == q && e.z == z) {
            *rl = e.rl;
            *rr = e.rr;
            return;
        }
    }
    RankMemo& e = g_rank_memo[g_rank_next];
    g_rank_next = (g_rank_next + 1) % 8;
    e.m = m;
    e.q = q;
    e.z = z;
    e.rl = lower_rank_exact(m, q, z);
    e.rr = upper_rank_exact(m, q, z);
    e.used = true;
    *rl = e.rl;
    *rr = e.rr;
}

int64_t lower_rank(int64_t m, double q, double z)
{
    int64_t a, b;
    bracket_ranks(m, q, z, &a, &b);
    return a;
}

int64_t upper_rank(int64_t m, double q, double z)
{
    int64_t a, b;
    bracket_ranks(m, q, z, &a, &b);
    return b;
}

int32_t filter_groups(int32_t m) { return (m + kFilterPer - 1) / kFilterPer; }

// Segment buffers from offset o (none below kSegMinN scores); returns the
// end.  One segment per wave share of every whole pass-1 tile.
int64_t seg_count(int64_t n)
{
    // four segments per whole large VJP tile (the emission's tiles too)
    const int64_t tiles = (n / 4) / (kVjpBatchLarge * kStreamThreads);
    return n >= kSegMinN ? tiles * (kStreamThreads / kWave) : 0;
}

size_t seg_layout(int64_t n, size_t o, int64_t* n_seg, size_t* off_cnt, size_t* off_ent)
{
    const int64_t segs = seg_count(n);
    *n_seg = segs;
    *off_cnt = o;
    o = align_up(o + sizeof(uint32_t) * (size_t)segs);
    *off_ent = o;
    o = align_up(o + sizeof(uint64_t) * kSegCap * (size_t)segs);
    return o;
}

// The segment buffers of a forward workspace at ws (all null when unused).
SegBufs seg_bufs(char* ws, int64_t n_seg, size_t off_cnt, size_t off_ent)
{
    SegBufs b;
    b.cnt = nullptr;
    b.ent = nullptr;
    if (n_seg > 0) {
        b.cnt = reinterpret_cast<uint32_t*>(ws + off_cnt);
        b.ent = reinterpret_cast<uint64_t*>(ws + off_ent);
    }
    return b;
}

uint32_t host_key(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct Ctx {
    const float* s;
    int64_t n;
    double k, alpha, c;
    float* p;
    double* b;
    char* ws;
    Plan plan;
    hipStream_t stream;
    Status* st;
    uint64_t seed;
    Mirror* mirror0;   // device address of host mirror slot 0 (solve)
    Mirror* mirror1;   // device address of host mirror slot 1 (mass fold)
    bool count_only = false;  // this round's pass-1 keeps no band (expected to overflow)
};

// Two status mirrors per host thread in pinned, fine-grained host memory:
// slot 0 is written by the segment solve as it finishes (the bracket
// certificate), slot 1 by the fold of the certification pass (the fp64 mass).
// A solve publishes slot 0 with a sequence number of its own, written after
// a system-scope release: the host spins on that number instead of waiting
// for an event, so nothing is recorded on the stream between the solve and
// the emission (an event there costs the GPU a few microseconds between the
// two kernels).  Slot 1, and a plain copy into slot 0 for the rare reads
// that follow no solve (the score range of the full-sort route), are each
// followed by an event the host waits on without draining the stream.
struct HostSlots {
    Mirror* pinned = nullptr;
    hipEvent_t ev[2] = {nullptr, nullptr};
    uint32_t seq = 0;      // last publication number handed out
};
thread_local HostSlots g_host;

int ensure_host_slots()
{
    if (!g_host.pinned) {
        void* ptr = nullptr;
        STK_HIP(hipHostMalloc(&ptr, 2 * sizeof(Mirror), hipHostMallocCoherent | hipHostMallocMapped | hipHostMallocPortable));
        memset(ptr, 0, 2 * sizeof(Mirror));
        g_host.pinned = static_cast<Mirror*>(ptr);
        for (int i = 0; i < 2; ++i)
            STK_HIP(hipEventCreateWithFlags(&g_host.ev[i], hipEventDisableTiming));
    }
    return SOFT_TOPK_OK;
}

// Device-usable address of a mirror slot.
Mirror* mirror_slot(int slot)
{
    void* dev = nullptr;
    if (hipHostGetDevicePointer(&dev, g_host.pinned, 0) != hipSuccess || dev == nullptr)
        return nullptr;
    return static_cast<Mirror*>(dev) + slot;
}

// The number the next solve publishes slot 0 with (never 0).
uint32_t next_publication()
{
    if (++g_host.seq == 0u)
        g_host.seq = 1u;
    return g_host.seq;
}

int mark_status(const Ctx& x, int slot)
{
    STK_HIP(hipEventRecord(g_host.ev[slot], x.stream));
    return SOFT_TOPK_OK;
}

int enqueue_status_copy(const Ctx& x, int slot)
{
    int rc = ensure_host_slots();
    if (rc)
        return rc;
    STK_HIP(hipMemcpyAsync(&g_host.pinned[slot].st, x.st, sizeof(Status), hipMemcpyDeviceToHost, x.stream));
    return mark_status(x, slot);
}

int wait_status(int slot, Status* host)
{
    STK_HIP(hipEventSynchronize(g_host.ev[slot]));
    memcpy(host, &g_host.pinned[slot].st, sizeof(Status));
    return SOFT_TOPK_OK;
}

// Wait for the last solve's publication of slot 0.  The stream is queried
// now and then: an error on it is returned, and a stream that has drained
// without the publication (which cannot happen short of an error) is one.
int wait_solve(const Ctx& x, Status* host)
{
    const uint32_t want = g_host.seq;
    const uint32_t* seq = &g_host.pinned[0].seq;
    for (uint32_t spins = 1; __atomic_load_n(seq, __ATOMIC_ACQUIRE) != want; ++spins) {
        if ((spins & 1023u) == 0u) {
            const hipError_t e = hipStreamQuery(x.stream);
            if (e == hipSuccess) {
                if (__atomic_load_n(seq, __ATOMIC_ACQUIRE) == want)
                    break;
                return hip_fail(hipErrorLaunchFailure);
            }
            if (e != hipErrorNotReady)
                return hip_fail(e);
        }
        __builtin_ia32_pause();
    }
    memcpy(host, const_cast<const Status*>(&g_host.pinned[0].st), sizeof(Status));
    return SOFT_TOPK_OK;
}

int read_status(const Ctx& x, Status* host)
{
    int rc = enqueue_status_copy(x, 0);
    if (rc)
        return rc;
    return wait_status(0, host);
}

template <typename T>
T* at(const Ctx& x, size_t off)
{
    return reinterpret_cast<T*>(x.ws + off);
}

int enqueue_pass1(const Ctx& x)
{
    Pass1Args a;
    a.s = x.s;
    a.n = x.n;
    a.log2e_over_alpha = x.c;
    a.band = at<float>(x, x.plan.off_band);
    a.cap = x.plan.cap;
    a.partials = at<Pass1Partial>(x, x.plan.off_p1part);
    a.blocks = x.plan.g_pass1;
    a.count_only = x.count_only ? 1 : 0;
    a.st = x.st;
    STK_HIP(launch_pass1(a, x.stream));
    return SOFT_TOPK_OK;
}

int enqueue_emit(const Ctx& x, bool fold_mass)
{
    EmitArgs e;
    e.s = x.s;
    e.n = x.n;
    e.alpha = x.alpha;
    e.log2e_over_alpha = x.c;
    e.b = x.b;
    e.p = x.p;
    e.partials = at<double>(x, x.plan.off_emitpart);
    e.blocks = x.plan.g_emit;
    e.st = x.st;
    e.mirror = x.mirror1;
    e.seg = seg_bufs(x.ws, x.plan.n_seg, x.plan.off_seg_cnt, x.plan.off_seg_ent);
    STK_HIP(launch_emit(e, fold_mass, x.stream));
    return SOFT_TOPK_OK;
}

// Band sort (unless the band is sorted whole) and the segment solve of a
// bracketed round whose pass-1 has been enqueued.
int enqueue_band_solve(const Ctx& x, bool direct)
{
    BandArgs ba;
    ba.p1 = at<Pass1Partial>(x, x.plan.off_p1part);
    ba.p1_blocks = x.plan.g_pass1;
    ba.p1_super = at<Pass1Partial>(x, x.plan.off_super);
    ba.band = at<float>(x, x.plan.off_band);
    ba.band_sorted = at<float>(x, x.plan.off_band_sorted);
    ba.cap = x.plan.cap;
    ba.hist = at<uint32_t>(x, x.plan.off_hist);
    ba.bstart = at<uint32_t>(x, x.plan.off_bstart);
    ba.agg = at<GroupAgg>(x, x.plan.off_agg);
    ba.blocks = x.plan.g_band;
    ba.log2e_over_alpha = x.c;
    ba.st = x.st;
    if (!direct)
        STK_HIP(launch_band_sort(ba, x.stream));
    SolveArgs so;
    so.p1 = ba.p1;
    so.p1_blocks = ba.p1_blocks;
    so.p1_super = ba.p1_super;
    so.sorted = direct ? ba.band : ba.band_sorted;
    so.agg = ba.agg;
    so.scan = at<GroupScan>(x, x.plan.off_scan);
    so.groups = direct ? 0 : kBuckets;
    so.tails = 1;
    so.direct = direct ? 1 : 0;
    so.cap = x.plan.cap;
    so.k = x.k;
    so.alpha = x.alpha;
    so.log2e_over_alpha = x.c;
    so.out_b = x.b;
    so.st = x.st;
    so.mirror = x.mirror0;
    so.seq = next_publication();
    STK_HIP(launch_solve(so, x.stream));
    return SOFT_TOPK_OK;
}

// The band's expected size for sample ranks (rl, rr): n (rr - rl) / m, or
// infinity when a bracket end is open.
double band_predict(int64_t n, int64_t m, int64_t rl, int64_t rr)
{
    if (rl < 1 || rr > m)
        return INFINITY;
    return (double)n * (double)(rr - rl) / (double)m;
}

// Whether a sorted round with sample ranks (rl, rr) sorts its band whole:
// both bracket ends finite and the expected band small enough.
bool band_direct(const soft_topk_params& prm, int64_t n, int64_t m, int64_t rl, int64_t rr)
{
    if (prm.band_route == SOFT_TOPK_BAND_BUCKETS)
        return false;
    if (prm.band_route == SOFT_TOPK_BAND_DIRECT)
        return true;
    return band_predict(n, m, rl, rr) <= kDirectPredictMax;
}

// Step kernels per chain: the most passes any of the last kHintCalls chains
// took (within kIterStepsMin..kIterStepsMax).  Each launch costs 4-5 us
// whatever it does, so a chain longer than needed costs that much per
// extra step; one that runs out resumes where it stopped.
constexpr int kHintCalls = 4;
thread_local int g_chain_passes[kHintCalls] = {3, 3, 3, 3};
thread_local int g_chain_next = 0;

int chain_steps()
{
    int m = kIterStepsMin;
    for (int v : g_chain_passes)
        m = std::max(m, v);
    return std::min(m, kIterStepsMax);
}

void note_chain_passes(int passes)
{
    g_chain_passes[g_chain_next] = passes;
    g_chain_next = (g_chain_next + 1) % kHintCalls;
}

// The last (n, k, alpha, band capacity) on this thread whose first
// bracket's band overflowed its buffer.  A call with the same shape expects the same (a
// tied cluster at the threshold stays there from batch to batch): its
// pass-1 only counts the band, since filling a buffer that overflows costs
// one serialised reservation per 512 band scores, and every score is
// refined.  The count is exact, so a band that turns out to fit clears the
// hint for the next call; the result is exact either way.
struct OverflowHint {
    int64_t n = 0, cap = 0;
    double k = 0.0, alpha = 0.0;
};
thread_local OverflowHint g_overflow;

bool overflow_expected(int64_t n, int64_t cap, double k, double alpha)
{
    return g_overflow.n == n && g_overflow.cap == cap && g_overflow.k == k && g_overflow.alpha == alpha;
}

void note_overflow(int64_t n, int64_t cap, double k, double alpha, bool overflowed)
{
    if (overflowed)
        g_overflow = OverflowHint{n, cap, k, alpha};
    else if (overflow_expected(n, cap, k, alpha))
        g_overflow = OverflowHint{};
}

// Partition refinement of the band (or of every score when the band
// overflowed): one work-group, or a chain of `steps` step kernels (resume:
// from where the last chain stopped, after passes_before passes).
int enqueue_refine(const Ctx& x, bool one_group, int steps, bool resume, int passes_before)
{
    IterArgs ia;
    ia.band = at<float>(x, x.plan.off_band);
    ia.cap = x.count_only ? 0 : x.plan.cap;  // no band kept: every score is refined (unless none is in it)
    ia.s = x.s;
    ia.n = x.n;
    ia.p1 = at<Pass1Partial>(x, x.plan.off_p1part);
    ia.p1_blocks = x.plan.g_pass1;
    ia.is = at<IterState>(x, x.plan.off_iter);
    ia.part = at<SplitPartial>(x, x.plan.off_iter + align_up(sizeof(IterState)));
    ia.groups = x.count_only ? kIterGroupsAll : kIterGroups;  // every score refined: a wider grid
    ia.passes_before = passes_before;
    ia.k = x.k;
    ia.alpha = x.alpha;
    ia.log2e_over_alpha = x.c;
    ia.out_b = x.b;
    ia.st = x.st;
    ia.mirror = x.mirror0;
    ia.seq = next_publication();
    STK_HIP(launch_partition_solve(ia, one_group, steps, resume, x.stream));
    return SOFT_TOPK_OK;
}

// How a round solves its band: refinement (on one work-group when the band
// is expected to fit it, else by the step kernels), or one of the sorted
// routes when the parameters force it.
int round_route(const soft_topk_params& prm, int64_t n, int64_t m, int64_t rl, int64_t rr)
{
    if (prm.band_route == SOFT_TOPK_BAND_DIRECT || prm.band_route == SOFT_TOPK_BAND_BUCKETS)
        return band_direct(prm, n, m, rl, rr) ? SOFT_TOPK_BAND_DIRECT : SOFT_TOPK_BAND_BUCKETS;
    if (prm.band_route == SOFT_TOPK_BAND_REFINE_STEPS)
        return SOFT_TOPK_BAND_REFINE_STEPS;
    return band_predict(n, m, rl, rr) <= kIterOnePredictMax ? SOFT_TOPK_BAND_REFINE : SOFT_TOPK_BAND_REFINE_STEPS;
}

// One bracketed round: select with ranks (rl, rr), pass-1, then the band's
// solve by `route`.
int enqueue_round(const Ctx& x, int64_t rl, int64_t rr, double q, int route)
{
    SampleArgs sa;
    sa.s = x.s;
    sa.n = x.n;
    sa.alpha = (float)x.alpha;
    sa.k0 = (uint32_t)(x.seed & 0xffffffffu);
    sa.k1 = (uint32_t)(x.seed >> 32);
    sa.m = x.plan.m;
    sa.r_left = rl;
    sa.r_right = rr;
    sa.q = q;
    sa.cand = at<uint32_t>(x, x.plan.off_samples);
    sa.rec = at<FilterRec>(x, x.plan.off_frec);
    SelectArgs se;
    se.cand = sa.cand;
    se.rec = sa.rec;
    se.groups = filter_groups(x.plan.m);
    se.m = x.plan.m;
    se.r_left = rl;
    se.r_right = rr;
    se.st = x.st;
    STK_HIP(launch_localize(sa, se, x.stream));
    int rc = enqueue_pass1(x);
    if (rc)
        return rc;
    if (route == SOFT_TOPK_BAND_REFINE || route == SOFT_TOPK_BAND_REFINE_STEPS)
        return enqueue_refine(x, route == SOFT_TOPK_BAND_REFINE, chain_steps(), false, 0);
    return enqueue_band_solve(x, route == SOFT_TOPK_BAND_DIRECT);
}

// Radix sort of all scores and summaries of 4096-score tiles of the sorted
// values (which replace the keys in place).  Returns the sorted values.
int enqueue_sorted_tiles(const Ctx& x, const Status& range, const float** sorted_values)
{
    // sort only the key bits that vary between the smallest and largest score
    const uint32_t kmin = host_key(range.smin);
    const uint32_t span = host_key(range.smax) - kmin;
    int bits = 0;
    while (bits < 32 && (span >> bits) != 0)
        ++bits;
    const int passes = std::max(1, (bits + 7) / 8);
    RadixArgs ra;
    ra.s = x.s;
    ra.n = x.n;
    ra.keys0 = at<uint32_t>(x, x.plan.off_keys0);
    ra.keys1 = at<uint32_t>(x, x.plan.off_keys1);
    ra.hist = at<uint32_t>(x, x.plan.off_rhist);
    ra.g_radix = x.plan.g_radix;
    ra.key_min = kmin;
    ra.passes = passes;
    ra.st = x.st;
    uint32_t* sorted = nullptr;
    ra.sorted_out = &sorted;
    STK_HIP(launch_radix_sort(ra, x.stream));
    TileArgs ta;
    ta.keys = sorted;
    ta.n = x.n;
    ta.key_min = kmin;
    ta.agg = at<GroupAgg>(x, x.plan.off_agg);
    ta.n_tiles = x.plan.n_tiles;
    ta.log2e_over_alpha = x.c;
    STK_HIP(launch_tile_aggregates(ta, x.stream));
    *sorted_values = reinterpret_cast<const float*>(sorted);
    return SOFT_TOPK_OK;
}

int enqueue_fullsort(const Ctx& x, const Status& range)
{
    const float* sorted = nullptr;
    int rc = enqueue_sorted_tiles(x, range, &sorted);
    if (rc)
        return rc;
    SolveArgs so;
    so.p1 = nullptr;
    so.p1_blocks = 0;
    so.p1_super = nullptr;
    so.sorted = sorted;
    so.agg = at<GroupAgg>(x, x.plan.off_agg);
    so.scan = at<GroupScan>(x, x.plan.off_scan);
    so.groups = x.plan.n_tiles;
    so.tails = 0;
    so.direct = 0;
    so.cap = x.plan.cap;
    so.k = x.k;
    so.alpha = x.alpha;
    so.log2e_over_alpha = x.c;
    so.out_b = x.b;
    so.st = x.st;
    so.mirror = x.mirror0;
    so.seq = next_publication();
    STK_HIP(launch_solve(so, x.stream));
    return SOFT_TOPK_OK;
}

// After a solve (which publishes mirror slot 0 as it finishes): enqueue the
// emission with its per-work-group fp64 sums of p.  When the mass is to be
// waited for, also enqueue the fold of those sums (which writes slot 1) and
// mark slot 1.
int enqueue_certify_emit(const Ctx& x, bool wait_mass)
{
    int rc = enqueue_emit(x, wait_mass);
    if (rc)
        return rc;
    return wait_mass ? mark_status(x, 1) : SOFT_TOPK_OK;
}

bool mass_ok(const Status& h, double k, double tol)
{
    return h.emit_done && fabs(h.mass - k) <= tol;
}

// b strictly between the tied value T and the next float T+ (the round
// above T rejected low, M(T+) < k, and the round below rejected high,
// M(T) > k): the closed form in the gap right of T runs on the device
// (tie_root_kernel), from the first round's left tail (kept in the status
// block when the second round's bracket was set) and the second round's
// right tail, and publishes the status like a segment solve.
int tie_root(const Ctx& x, bool wait_mass, double tol, soft_topk_stats* sx, Status* h, bool* done)
{
    TieRootArgs ta;
    ta.st = x.st;
    ta.out_b = x.b;
    ta.n = x.n;
    ta.k = x.k;
    ta.alpha = x.alpha;
    ta.log2e_over_alpha = x.c;
    ta.mirror = x.mirror0;
    ta.seq = next_publication();
    STK_HIP(launch_tie_root(ta, x.stream));
    int rc = enqueue_certify_emit(x, wait_mass);
    if (rc)
        return rc;
    rc = wait_solve(x, h);
    if (rc)
        return rc;
    if (h->solve_state != kSolveOk)
        return SOFT_TOPK_OK;
    if (wait_mass) {
        rc = wait_status(1, h);
        if (rc)
            return rc;
        if (!mass_ok(*h, x.k, tol)) {
            sx->reject_mask |= SOFT_TOPK_REJECT_MASS;
            return SOFT_TOPK_OK;
        }
    }
    sx->path = SOFT_TOPK_PATH_WIDENED;
    *done = true;
    return SOFT_TOPK_OK;
}

// A band (or a band bucket) too large to sort because one value fills a
// large part of it: a cluster of exact ties that every bracket around b
// contains when b lies among them.  Split the bracket at that value T: on
// [T+, a_R) the whole cluster lies in the left tail, on [a_L, T) in the right
// tail, and either band holds only the other scores near b.  The side above
// T is tried first; the certificate of each round decides.  When the first
// rejects low and the second high, b lies between T and T+ (tie_root).  No
// dominant value, or any other outcome, leaves the full sort to decide.
// Uses at most `rounds_left` more rounds.
int tie_split(const Ctx& x, Status h0, int rounds_left, bool wait_mass, double tol, soft_topk_stats* sx, Status* h,
              bool* done)
{
    // the band histogram region is free until the next round's band sort
    STK_HIP(launch_band_mode(at<float>(x, x.plan.off_band), x.plan.cap, x.st, at<uint32_t>(x, x.plan.off_hist),
                             x.stream));
    int rc = read_status(x, h);
    if (rc)
        return rc;
    const int64_t m = std::min<int64_t>((int64_t)h0.nB, x.plan.cap);
    if ((int64_t)h->tie_count < std::max<int64_t>(m / 8, 1024))
        return SOFT_TOPK_OK;
    const float T = h->tie_value;
    const float Tp = nextafterf(T, INFINITY);
    const float br[2][2] = {{Tp, h0.aR > Tp ? h0.aR : INFINITY}, {h0.aL < T ? h0.aL : -INFINITY, T}};
    bool above_low = false;
    for (int i = 0; i < 2 && i < rounds_left; ++i) {
        // the second round keeps the first round's left tail for tie_root
        STK_HIP(launch_set_bracket(x.st, br[i][0], br[i][1], i == 1, x.stream));
        rc = enqueue_pass1(x);
        if (rc)
            return rc;
        rc = enqueue_band_solve(x, false);
        if (rc)
            return rc;
        rc = enqueue_certify_emit(x, wait_mass);
        if (rc)
            return rc;
        rc = wait_solve(x, h);
        if (rc)
            return rc;
        sx->rounds += 1;
        sx->band_route = SOFT_TOPK_BAND_BUCKETS;
        sx->refine_passes = 0;
        sx->a_left = h->aL;
        sx->a_right = h->aR;
        sx->n_left = (int64_t)h->nL;
        sx->n_right = (int64_t)h->nR;
        sx->n_band = (int64_t)h->nB;
        sx->mass_at_left = h->massL;
        sx->mass_at_right = h->massR;
        if (h->nonfinite)
            return SOFT_TOPK_ENONFINITE;
        if (h->solve_state == kSolveOk) {
            if (wait_mass) {
                rc = wait_status(1, h);
                if (rc)
                    return rc;
            }
            if (!wait_mass || mass_ok(*h, x.k, tol)) {
                sx->path = SOFT_TOPK_PATH_WIDENED;
                *done = true;
            } else {
                sx->reject_mask |= SOFT_TOPK_REJECT_MASS;
            }
            return SOFT_TOPK_OK;
        }
        if (h->solve_state == kSolveRejectLow) {
            sx->reject_mask |= SOFT_TOPK_REJECT_LOW;  // b < T+: the side below
            if (i == 0)
                above_low = true;
            continue;
        }
        if (h->solve_state == kSolveRejectHigh) {
            sx->reject_mask |= SOFT_TOPK_REJECT_HIGH;
            if (i == 1 && above_low)
                return tie_root(x, wait_mass, tol, sx, h, done);
        } else if (h->solve_state == kSolveOverflow) {
            sx->reject_mask |= SOFT_TOPK_REJECT_OVERFLOW;
        } else if (h->solve_state == kSolveBucketOverflow) {
            sx->reject_mask |= SOFT_TOPK_REJECT_BUCKET;
        }
        return SOFT_TOPK_OK;
    }
    return SOFT_TOPK_OK;
}

// After a refining round: a band larger than the one-work-group form, or
// than its buffer, is refined by the step kernels (every score, when it
// overflowed); a band refinement that did not end falls back to sorting the
// band; every score refined without an end counts as a band overflow (the
// tie split and the full sort follow).  Each follow-up is one more solve
// and emission on the same pass-1 output.  *route becomes the route that
// ran last.
int settle_refine(const Ctx& x, bool direct, bool wait_mass, Status* h, int* route)
{
    int rc;
    if (*route == SOFT_TOPK_BAND_REFINE && (h->solve_state == kSolveIterBig || h->solve_state == kSolveOverflow)) {
        *route = SOFT_TOPK_BAND_REFINE_STEPS;
        rc = enqueue_refine(x, false, chain_steps(), false, 0);
        if (rc)
            return rc;
        rc = enqueue_certify_emit(x, wait_mass);
        if (rc)
            return rc;
        rc = wait_solve(x, h);
        if (rc)
            return rc;
    }
    // a chain that ran out of steps resumes where it stopped
    while (h->solve_state == kSolveIterMore && (int)h->iter_steps < kIterPassesMax) {
        rc = enqueue_refine(x, false, kIterStepsMax, true, (int)h->iter_steps);
        if (rc)
            return rc;
        rc = enqueue_certify_emit(x, wait_mass);
        if (rc)
            return rc;
        rc = wait_solve(x, h);
        if (rc)
            return rc;
    }
    if (*route == SOFT_TOPK_BAND_REFINE_STEPS && h->solve_state != kSolveNonfinite)
        note_chain_passes((int)h->iter_steps);
    if (h->solve_state == kSolveIterMore)
        h->solve_state = kSolveIterLimit;
    if (h->solve_state != kSolveIterLimit)
        return SOFT_TOPK_OK;
    if (h->iter_mode == 1u) {
        h->solve_state = kSolveOverflow;
        return SOFT_TOPK_OK;
    }
    *route = direct ? SOFT_TOPK_BAND_DIRECT : SOFT_TOPK_BAND_BUCKETS;
    for (int i = 0; i < 2; ++i) {
        rc = enqueue_band_solve(x, direct);
        if (rc)
            return rc;
        rc = enqueue_certify_emit(x, wait_mass);
        if (rc)
            return rc;
        rc = wait_solve(x, h);
        if (rc)
            return rc;
        if (h->solve_state != kSolveDirectOverflow)
            break;
        direct = false;  // the band outgrew the whole-band sort: bucket it
        *route = SOFT_TOPK_BAND_BUCKETS;
    }
    return SOFT_TOPK_OK;
}

}  // namespace

Plan make_plan(int64_t n, int32_t m, int64_t cap)
{
    Plan p;
    memset(&p, 0, sizeof(p));
    p.n = n;
    p.m = m;
    p.cap = cap;
    p.g_pass1 = pass1_blocks(n);
    p.g_emit = emit_blocks(n);
    p.g_band = kBandGroups;
    p.n_tiles = (int32_t)((n + kTile - 1) / kTile);
    p.g_radix = (int32_t)((n + kRadixTile - 1) / kRadixTile);
    const int64_t groups = std::max<int64_t>(kBuckets, p.n_tiles);
    size_t o = 0;
    p.off_status = o;
    o = align_up(o + sizeof(Status));
    // saturated-score segments first: their place depends on n alone, so the
    // backward can find them in a forward workspace
    o = seg_layout(n, o, &p.n_seg, &p.off_seg_cnt, &p.off_seg_ent);
    p.off_samples = o;  // candidate keys of the localisation, one region per filter group
    o = align_up(o + sizeof(uint32_t) * (size_t)filter_groups(m) * kFilterPer);
    p.off_frec = o;
    o = align_up(o + sizeof(FilterRec) * (size_t)filter_groups(m));
    p.off_p1part = o;
    o = align_up(o + sizeof(Pass1Partial) * (size_t)p.g_pass1);
    p.off_band = o;
    o = align_up(o + sizeof(float) * (size_t)cap);
    p.off_band_sorted = o;
    o = align_up(o + sizeof(float) * (size_t)cap);
    p.off_hist = o;
    o = align_up(o + sizeof(uint32_t) * (size_t)p.g_band * kBuckets);
    p.off_bstart = o;
    o = align_up(o + sizeof(uint32_t) * (kBuckets + 1));
    p.off_agg = o;
    o = align_up(o + sizeof(GroupAgg) * (size_t)groups);
    p.off_scan = o;
    o = align_up(o + sizeof(GroupScan) * (size_t)groups);
    p.off_emitpart = o;
    o = align_up(o + sizeof(double) * (size_t)p.g_emit);
    p.off_iter = o;
    o = align_up(o + align_up(sizeof(IterState)) + sizeof(SplitPartial) * 2 * (size_t)kIterGroupsAll);
    p.off_keys0 = o;
    o = align_up(o + sizeof(uint32_t) * (size_t)n);
    p.off_keys1 = o;
    o = align_up(o + sizeof(uint32_t) * (size_t)n);
    p.off_rhist = o;
    // [tile][digit] counts (turned into offsets in place), then the chunk sums
    o = align_up(o + sizeof(uint32_t) * kRadixBins * ((size_t)p.g_radix + kRadixMaxChunks));
    p.off_super = o;
    o = align_up(o + sizeof(Pass1Partial) * (size_t)kBuckets);
    p.total = o;
    return p;
}

}  // namespace stk

using namespace stk;

// ---- scratch of the allocation-free backward ------------------------------
// The score-reading backward needs one buffer beyond its inputs and outputs:
// the (D, G) partials of its reduction, one fp64 pair per work-group.  Its
// grid is capped at kNoAllocPartials work-groups for every n, so a fixed
// device array holds them.  Each GPU the library runs on holds its own copy
// (16 KiB) until the process ends; its address is looked up once per device.
constexpr int kNoAllocPartials = 1024;
static_assert(kGridVjpLarge <= kNoAllocPartials && kGridVjpSmall <= kNoAllocPartials,
              "the score-reading reduction grid must fit the fixed scratch");
static __device__ __align__(256) double scratch[2 * kNoAllocPartials];

namespace {

bool n_ok(int64_t n) { return n >= 1 && n <= 0x7fffffffLL; }

constexpr int kMaxDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    double* ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of `scratch` on the current device (the host-side name is a
// stand-in, not a device address: only this pointer reaches kernels).
int scratch_on_current_device(double** out)
{
    int dev = -1;
    STK_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices)
        return hip_fail(hipErrorInvalidDevice);
    ScratchSlot& slot = g_scratch[dev];
    std::call_once(slot.once, [&slot]() {
        void* p = nullptr;
        slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (slot.err == hipSuccess && p == nullptr)
            slot.err = hipErrorInvalidSymbol;
        slot.ptr = static_cast<double*>(p);
    });
    if (slot.err != hipSuccess)
        return hip_fail(slot.err);
    *out = slot.ptr;
    return SOFT_TOPK_OK;
}

bool rows_ok(int64_t rows, int64_t n_row)
{
    return rows >= 1 && n_row >= 1 && rows <= 0x7fffffffLL && n_ok(n_row) && rows <= INT64_MAX / n_row;
}

RowsArgs rows_args(const float* s, int64_t rows, int64_t n_row, double alpha)
{
    RowsArgs a;
    memset(&a, 0, sizeof(a));
    a.s = s;
    a.rows = rows;
    a.n_row = (int32_t)n_row;
    a.alpha = alpha;
    a.log2e_over_alpha = kLog2e / alpha;
    return a;
}


soft_topk_params resolve(const soft_topk_params* params)
{
    soft_topk_params p;
    fill_defaults(&p);
    if (params)
        p = *params;
    return p;
}

Plan plan_for(int64_t n, const soft_topk_params& p)
{
    const int64_t cap = p.band_capacity > 0 ? std::min<int64_t>(p.band_capacity, n) : default_cap(n);
    return make_plan(n, p.samples, cap);
}

}  // namespace

extern "C" {

void soft_topk_default_params(soft_topk_params* params)
{
    if (params)
        fill_defaults(params);
}

size_t soft_topk_workspace_bytes(int64_t n, const soft_topk_params* params)
{
    if (!n_ok(n))
        return 0;
    const soft_topk_params p = resolve(params);
    if (!params_ok(p))
        return 0;
    return plan_for(n, p).total;
}

size_t soft_topk_record_bytes(int64_t n)
{
    if (!n_ok(n))
        return 0;
    int64_t n_seg;
    size_t off_cnt, off_ent;
    return seg_layout(n, align_up(sizeof(Status)), &n_seg, &off_cnt, &off_ent);
}

size_t soft_topk_backward_workspace_bytes(int64_t n)
{
    if (!n_ok(n))
        return 0;
    // the reduction partials, then the listed g values of the segments
    return align_up(sizeof(double) * 2 * (size_t)vjp_partial_blocks(n)) +
           align_up(sizeof(float) * kSegCap * (size_t)seg_count(n));
}

const char* soft_topk_strerror(int code)
{
    switch (code) {
    case SOFT_TOPK_OK:
        return "ok";
    case SOFT_TOPK_EINVAL:
        return "invalid argument";
    case SOFT_TOPK_ENONFINITE:
        return "a score is NaN or infinite";
    case SOFT_TOPK_EWORKSPACE:
        return "workspace missing, misaligned or too small";
    case SOFT_TOPK_EHIP:
        return "HIP runtime error";
    case SOFT_TOPK_ESOLVE:
        return "no route produced a certified threshold";
    default:
        return "unknown error";
    }
}

int soft_topk_last_hip_error(void) { return g_last_hip; }

int soft_topk_bracket_ranks(int64_t m, double q, double z, int64_t* r_left, int64_t* r_right)
{
    if (m < 1 || !(q > 0.0) || !(q < 1.0) || !(z > 0.0) || !isfinite(z) || !r_left || !r_right)
        return SOFT_TOPK_EINVAL;
    *r_left = lower_rank(m, q, z);
    *r_right = upper_rank(m, q, z);
    return SOFT_TOPK_OK;
}

int soft_topk_forward_ex(const float* scores, int64_t n, double k, double alpha, float* out_p,
                         double* out_b, void* workspace, size_t workspace_bytes, void* stream,
                         const soft_topk_params* params, soft_topk_stats* stats)
{
    if (!scores || !out_p || !out_b || !n_ok(n))
        return SOFT_TOPK_EINVAL;
    if (!(alpha > 0.0) || !isfinite(alpha) || !(k > 0.0) || !(k < (double)n) || !isfinite(k))
        return SOFT_TOPK_EINVAL;
    const soft_topk_params prm = resolve(params);
    if (!params_ok(prm))
        return SOFT_TOPK_EINVAL;
    const Plan plan = plan_for(n, prm);
    if (!workspace || workspace_bytes < plan.total || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
        return SOFT_TOPK_EWORKSPACE;

    Ctx x;
    x.s = scores;
    x.n = n;
    x.k = k;
    x.alpha = alpha;
    x.c = kLog2e / alpha;
    x.p = out_p;
    x.b = out_b;
    x.ws = static_cast<char*>(workspace);
    x.plan = plan;
    x.stream = static_cast<hipStream_t>(stream);
    x.st = reinterpret_cast<Status*>(x.ws + plan.off_status);
    x.seed = prm.seed;
    int hrc = ensure_host_slots();
    if (hrc)
        return hrc;
    x.mirror0 = mirror_slot(0);
    x.mirror1 = mirror_slot(1);
    if (!x.mirror0 || !x.mirror1)
        return SOFT_TOPK_EHIP;

    const double tol = prm.mass_tolerance > 0.0 ? prm.mass_tolerance : 1e-3 + 1e-12 * (double)n;
    soft_topk_stats sx;
    memset(&sx, 0, sizeof(sx));
    Status h;
    memset(&h, 0, sizeof(h));
    bool done = false;
    // the fp64 mass of the emitted p gates the return only on request (or
    // when the caller wants the stats); the exact bracket certificate always
    // does
    const bool wait_mass = prm.verify_mass != 0 || stats != nullptr;

    if (n <= kRowMax && prm.force_path == 0 && prm.band_route == 0) {
        // one kernel sorts the whole vector in registers and solves it
        // exactly (the full-sort solver, with no bracket to certify), then
        // folds the fp64 mass and publishes the status (up to 64 scores a
        // second kernel does that)
        RowsArgs ra = rows_args(scores, 1, n, alpha);
        ra.p = out_p;
        ra.b = out_b;
        ra.k = k;
        const uint32_t seq = next_publication();
        if (n > 64) {
            ra.st = x.st;
            ra.mirror = x.mirror0;
            ra.seq = seq;
        }
        STK_HIP(launch_row_alone(ra, true, x.stream));
        if (n <= 64) {
            SingleArgs sa;
            sa.p = out_p;
            sa.b = out_b;
            sa.n = n;
            sa.st = x.st;
            sa.mirror = x.mirror0;
            sa.seq = seq;
            STK_HIP(launch_single_status(sa, x.stream));
        }
        int rc = wait_solve(x, &h);
        if (rc)
            return rc;
        if (h.nonfinite)
            return SOFT_TOPK_ENONFINITE;
        sx.n_band = n;
        sx.a_left = -INFINITY;
        sx.a_right = INFINITY;
        sx.mass_at_left = (double)n;
        sx.mass_at_right = 0.0;
        if (prm.verify_mass == 0 || mass_ok(h, k, tol)) {
            sx.path = SOFT_TOPK_PATH_SINGLE;
            done = true;
        } else {
            sx.reject_mask |= SOFT_TOPK_REJECT_MASS;  // the full sort decides
        }
    }

    if (!done && prm.force_path != SOFT_TOPK_PATH_FULLSORT) {
        const double q = 1.0 - k / (double)n;
        int64_t rl = lower_rank(plan.m, q, prm.z);
        int64_t rr = upper_rank(plan.m, q, prm.z);
        for (int round = 0; round <= prm.max_widen && !done; ++round) {
            int route = round_route(prm, n, plan.m, rl, rr);
            const bool refine = route == SOFT_TOPK_BAND_REFINE || route == SOFT_TOPK_BAND_REFINE_STEPS;
            // a first bracket whose band overflowed on the last call of this
            // shape: count the band only and refine every score
            x.count_only = refine && round == 0 && overflow_expected(n, plan.cap, k, alpha);
            if (x.count_only)
                route = SOFT_TOPK_BAND_REFINE_STEPS;
            const bool counted_only = x.count_only;  // this round's band buffer holds nothing
            int rc = enqueue_round(x, rl, rr, q, route);
            if (rc)
                return rc;
            rc = enqueue_certify_emit(x, wait_mass);
            if (rc)
                return rc;
            rc = wait_solve(x, &h);
            if (rc)
                return rc;
            if (refine) {
                rc = settle_refine(x, band_direct(prm, n, plan.m, rl, rr), wait_mass, &h, &route);
                if (rc)
                    return rc;
                if (round == 0 && !h.nonfinite)
                    note_overflow(n, plan.cap, k, alpha, h.nB > (uint64_t)plan.cap);
                x.count_only = false;  // later rounds keep their bands
            } else if (h.solve_state == kSolveDirectOverflow) {
                // the band outgrew the whole-band sort: bucket the same band
                route = SOFT_TOPK_BAND_BUCKETS;
                rc = enqueue_band_solve(x, false);
                if (rc)
                    return rc;
                rc = enqueue_certify_emit(x, wait_mass);
                if (rc)
                    return rc;
                rc = wait_solve(x, &h);
                if (rc)
                    return rc;
            }
            const bool all_scores = route == SOFT_TOPK_BAND_REFINE_STEPS && h.iter_mode == 1u;
            sx.rounds = round + 1;
            sx.band_route = route;
            sx.refine_passes = route == SOFT_TOPK_BAND_REFINE || route == SOFT_TOPK_BAND_REFINE_STEPS
                                   ? (int32_t)h.iter_steps
                                   : 0;
            if (all_scores)
                sx.reject_mask |= SOFT_TOPK_REJECT_OVERFLOW;
            sx.a_left = h.aL;
            sx.a_right = h.aR;
            sx.n_left = (int64_t)h.nL;
            sx.n_right = (int64_t)h.nR;
            sx.n_band = (int64_t)h.nB;
            sx.mass_at_left = h.massL;
            sx.mass_at_right = h.massR;
            if (h.nonfinite)
                return SOFT_TOPK_ENONFINITE;
            if (h.solve_state == kSolveOk) {
                if (wait_mass) {
                    rc = wait_status(1, &h);
                    if (rc)
                        return rc;
                }
                if (!wait_mass || mass_ok(h, k, tol)) {
                    sx.path = all_scores ? SOFT_TOPK_PATH_ALL_SCORES
                              : round == 0 ? SOFT_TOPK_PATH_BRACKET
                                           : SOFT_TOPK_PATH_WIDENED;
                    done = true;
                    break;
                }
                sx.reject_mask |= SOFT_TOPK_REJECT_MASS;
                break;  // the certified b failed the mass check: full sort
            }
            if (h.solve_state == kSolveRejectLow) {
                sx.reject_mask |= SOFT_TOPK_REJECT_LOW;
                // b < a_L: the old lower end is now a proven upper end
                const double z2 = prm.z * (double)(2 << round);
                rr = rl;
                rl = lower_rank(plan.m, q, z2);
                if (rl >= rr)
                    rl = 0;
                continue;
            }
            if (h.solve_state == kSolveRejectHigh) {
                sx.reject_mask |= SOFT_TOPK_REJECT_HIGH;
                const double z2 = prm.z * (double)(2 << round);
                rl = rr;
                rr = upper_rank(plan.m, q, z2);
                if (rr <= rl)
                    rr = plan.m + 1;
                continue;
            }
            if (h.solve_state == kSolveOverflow)
                sx.reject_mask |= SOFT_TOPK_REJECT_OVERFLOW;
            else if (h.solve_state == kSolveBucketOverflow)
                sx.reject_mask |= SOFT_TOPK_REJECT_BUCKET;
            if ((h.solve_state == kSolveOverflow || h.solve_state == kSolveBucketOverflow) && round < prm.max_widen &&
                !counted_only) {
                // widening cannot shrink the band; a tied cluster in it can be
                // split off into a tail (found in the band buffer, which a
                // counted-only round left unwritten: the full sort decides)
                rc = tie_split(x, h, prm.max_widen - round, wait_mass, tol, &sx, &h, &done);
                if (rc)
                    return rc;
            }
            break;  // otherwise the full sort decides
        }
    }

    if (!done) {
        // full-sort route: score range (and finiteness), then the radix sort
        STK_HIP(launch_reset_status(x.st, x.stream, false));
        STK_HIP(launch_range(x.s, n, at<Pass1Partial>(x, plan.off_p1part), plan.g_pass1, x.stream));
        STK_HIP(launch_pass1_finalize(at<Pass1Partial>(x, plan.off_p1part), plan.g_pass1, x.st, x.stream));
        int rc = read_status(x, &h);
        if (rc)
            return rc;
        if (h.nonfinite)
            return SOFT_TOPK_ENONFINITE;
        rc = enqueue_fullsort(x, h);
        if (rc)
            return rc;
        rc = enqueue_certify_emit(x, wait_mass);
        if (rc)
            return rc;
        rc = wait_solve(x, &h);
        if (rc)
            return rc;
        if (h.solve_state != kSolveOk)
            return SOFT_TOPK_ESOLVE;
        if (wait_mass) {
            rc = wait_status(1, &h);
            if (rc)
                return rc;
            if (!mass_ok(h, k, tol))
                return SOFT_TOPK_ESOLVE;
        }
        sx.path = SOFT_TOPK_PATH_FULLSORT;
    }
    sx.b = h.b;
    sx.mass = wait_mass ? h.mass : NAN;
    if (stats)
        *stats = sx;
    return SOFT_TOPK_OK;
}

int soft_topk_threshold_curve(const float* scores, int64_t n, double alpha, float* out_sorted, double* out_mass,
                              void* workspace, size_t workspace_bytes, void* stream)
{
    if (!scores || !out_sorted || !out_mass || !n_ok(n))
        return SOFT_TOPK_EINVAL;
    if (!(alpha > 0.0) || !isfinite(alpha))
        return SOFT_TOPK_EINVAL;
    const soft_topk_params prm = resolve(nullptr);
    const Plan plan = plan_for(n, prm);
    if (!workspace || workspace_bytes < plan.total || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
        return SOFT_TOPK_EWORKSPACE;
    Ctx x;
    memset(&x, 0, sizeof(x));
    x.s = scores;
    x.n = n;
    x.alpha = alpha;
    x.c = kLog2e / alpha;
    x.ws = static_cast<char*>(workspace);
    x.plan = plan;
    x.stream = static_cast<hipStream_t>(stream);
    x.st = reinterpret_cast<Status*>(x.ws + plan.off_status);
    int rc = ensure_host_slots();
    if (rc)
        return rc;
    x.mirror0 = mirror_slot(0);
    x.mirror1 = mirror_slot(1);
    if (!x.mirror0 || !x.mirror1)
        return SOFT_TOPK_EHIP;
    // score range (and finiteness), the radix sort, tile summaries, then
    // the masses
    Status h;
    STK_HIP(launch_reset_status(x.st, x.stream, false));
    STK_HIP(launch_range(x.s, n, at<Pass1Partial>(x, plan.off_p1part), plan.g_pass1, x.stream));
    STK_HIP(launch_pass1_finalize(at<Pass1Partial>(x, plan.off_p1part), plan.g_pass1, x.st, x.stream));
    rc = read_status(x, &h);
    if (rc)
        return rc;
    if (h.nonfinite)
        return SOFT_TOPK_ENONFINITE;
    const float* sorted = nullptr;
    rc = enqueue_sorted_tiles(x, h, &sorted);
    if (rc)
        return rc;
    CurveArgs ca;
    ca.sorted = sorted;
    ca.agg = at<GroupAgg>(x, plan.off_agg);
    ca.ex = x.ws + plan.off_scan;
    ca.n = n;
    ca.n_tiles = plan.n_tiles;
    ca.log2e_over_alpha = x.c;
    ca.out_sorted = out_sorted;
    ca.out_mass = out_mass;
    STK_HIP(launch_curve(ca, x.stream));
    return SOFT_TOPK_OK;
}

int soft_topk_forward(const float* scores, int64_t n, double k, double alpha, float* out_p, double* out_b,
                      void* workspace, size_t workspace_bytes, void* stream)
{
    return soft_topk_forward_ex(scores, n, k, alpha, out_p, out_b, workspace, workspace_bytes, stream,
                                nullptr, nullptr);
}

int soft_topk_backward(const float* grad_p, const float* scores, int64_t n, double alpha, const double* b,
                       float* grad_s, void* workspace, size_t workspace_bytes, void* stream)
{
    return soft_topk_backward_ex(grad_p, scores, n, alpha, b, grad_s, nullptr, 0, workspace, workspace_bytes, stream);
}

int soft_topk_backward_ex(const float* grad_p, const float* scores, int64_t n, double alpha, const double* b,
                          float* grad_s, const void* fwd_workspace, size_t fwd_workspace_bytes, void* workspace,
                          size_t workspace_bytes, void* stream)
{
    if (fwd_workspace && (reinterpret_cast<uintptr_t>(fwd_workspace) % kAlign) != 0)
        return SOFT_TOPK_EWORKSPACE;
    if (!grad_p || !scores || !b || !grad_s || !n_ok(n))
        return SOFT_TOPK_EINVAL;
    if (!(alpha > 0.0) || !isfinite(alpha))
        return SOFT_TOPK_EINVAL;
    const size_t need = soft_topk_backward_workspace_bytes(n);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) % 16) != 0)
        return SOFT_TOPK_EWORKSPACE;
    if (n <= kRowMax) {
        // one work-group reduces D and G and writes the gradient (the row
        // kernel with one row)
        RowsArgs ra = rows_args(scores, 1, n, alpha);
        ra.g = grad_p;
        ra.b_in = b;
        ra.grad = grad_s;
        STK_HIP(launch_row_alone(ra, false, static_cast<hipStream_t>(stream)));
        return SOFT_TOPK_OK;
    }
    VjpArgs a;
    a.g = grad_p;
    a.s = scores;
    a.n = n;
    a.alpha = alpha;
    a.log2e_over_alpha = kLog2e / alpha;
    a.b = b;
    a.grad = grad_s;
    a.partials = static_cast<double*>(workspace);
    a.blocks = vjp_apply_blocks(n);
    a.reduce_blocks = vjp_reduce_blocks(n);
    a.fst = nullptr;
    a.seg = seg_bufs(nullptr, 0, 0, 0);
    a.seg_tiles = seg_count(n) / (kStreamThreads / kWave);
    a.gl = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    align_up(sizeof(double) * 2 * (size_t)vjp_partial_blocks(n)));
    if (fwd_workspace) {
        int64_t n_seg;
        size_t off_cnt, off_ent;
        const size_t end = seg_layout(n, align_up(sizeof(Status)), &n_seg, &off_cnt, &off_ent);
        if (n_seg > 0 && fwd_workspace_bytes >= end) {
            char* fw = static_cast<char*>(const_cast<void*>(fwd_workspace));
            a.fst = reinterpret_cast<const Status*>(fw);
            a.seg = seg_bufs(fw, n_seg, off_cnt, off_ent);
            a.reduce_blocks = seg_grid(n, kGridVjpSegReduce);
            a.blocks = seg_grid(n, kGridVjpSegApply);
        }
    }
    STK_HIP(launch_vjp(a, static_cast<hipStream_t>(stream)));
    return SOFT_TOPK_OK;
}

int soft_topk_backward_noalloc(const float* grad_p, const float* scores, int64_t n, double alpha, const double* b,
                               float* grad_s, void* stream)
{
    if (!grad_p || !scores || !b || !grad_s || !n_ok(n))
        return SOFT_TOPK_EINVAL;
    if (!(alpha > 0.0) || !isfinite(alpha))
        return SOFT_TOPK_EINVAL;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (n <= kRowMax) {
        // one work-group, no scratch (as soft_topk_backward)
        RowsArgs ra = rows_args(scores, 1, n, alpha);
        ra.g = grad_p;
        ra.b_in = b;
        ra.grad = grad_s;
        STK_HIP(launch_row_alone(ra, false, st));
        return SOFT_TOPK_OK;
    }
    const int32_t reduce_blocks = vjp_reduce_blocks(n);
    if (reduce_blocks > kNoAllocPartials)
        return SOFT_TOPK_EWORKSPACE;
    double* partials = nullptr;
    const int rc = scratch_on_current_device(&partials);
    if (rc)
        return rc;
    // the score-reading route of soft_topk_backward, with its partials in the
    // fixed scratch: every work-group of the reduction writes its pair before
    // the gradient kernel reads them, so nothing needs clearing
    VjpArgs a;
    a.g = grad_p;
    a.s = scores;
    a.n = n;
    a.alpha = alpha;
    a.log2e_over_alpha = kLog2e / alpha;
    a.b = b;
    a.grad = grad_s;
    a.partials = partials;
    a.blocks = vjp_apply_blocks(n);
    a.reduce_blocks = reduce_blocks;
    a.fst = nullptr;
    a.seg = seg_bufs(nullptr, 0, 0, 0);
    a.seg_tiles = 0;
    a.gl = nullptr;
    STK_HIP(launch_vjp(a, st));
    return SOFT_TOPK_OK;
}

namespace {

struct DftPlan {
    int32_t groups, g_emit;
    size_t off_status, off_state, off_totals, off_rows, off_emitpart, total;
};

DftPlan dft_plan(int64_t n)
{
    DftPlan p;
    const int64_t tiles = (n + kDftTileScores - 1) / kDftTileScores;
    p.groups = (int32_t)std::max<int64_t>(1, std::min<int64_t>(tiles, kDftMaxGroups));
    p.g_emit = emit_blocks(n);
    size_t o = 0;
    p.off_status = o;
    o = align_up(o + sizeof(Status));
    p.off_state = o;
    o = align_up(o + sizeof(DftState) * 3);
    p.off_totals = o;
    o = align_up(o + sizeof(uint32_t) * 3 * kDftRowWords);
    p.off_rows = o;
    o = align_up(o + sizeof(uint32_t) * (size_t)p.groups * kDftRowWords);
    p.off_emitpart = o;
    o = align_up(o + sizeof(double) * (size_t)p.g_emit);
    p.total = o;
    return p;
}

}  // namespace

size_t soft_topk_dftopk_workspace_bytes(int64_t n)
{
    if (n < 2 || !n_ok(n))
        return 0;
    return dft_plan(n).total;
}

int soft_topk_dftopk_forward(const float* scores, int64_t n, double k, double alpha, float* out_p, double* out_b,
                             double* out_mass, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!scores || !out_p || !out_b || n < 2 || !n_ok(n))
        return SOFT_TOPK_EINVAL;
    if (!(alpha > 0.0) || !isfinite(alpha) || !(k >= 1.0) || !(k <= (double)(n - 1)) || k != floor(k))
        return SOFT_TOPK_EINVAL;
    const DftPlan plan = dft_plan(n);
    if (!workspace || workspace_bytes < plan.total || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
        return SOFT_TOPK_EWORKSPACE;
    char* ws = static_cast<char*>(workspace);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    Status* status = reinterpret_cast<Status*>(ws + plan.off_status);
    DftArgs a;
    a.s = scores;
    a.n = n;
    a.k = (int64_t)k;
    a.rows = reinterpret_cast<uint32_t*>(ws + plan.off_rows);
    a.totals = reinterpret_cast<uint32_t*>(ws + plan.off_totals);
    a.state = reinterpret_cast<DftState*>(ws + plan.off_state);
    a.groups = plan.groups;
    a.st = status;
    a.out_b = out_b;
    STK_HIP(launch_dftopk_threshold(a, st));
    EmitArgs e;
    e.s = scores;
    e.n = n;
    e.alpha = alpha;
    e.log2e_over_alpha = kLog2e / alpha;
    e.b = out_b;
    e.p = out_p;
    e.partials = reinterpret_cast<double*>(ws + plan.off_emitpart);
    e.blocks = plan.g_emit;
    e.st = status;
    e.mirror = nullptr;
    e.seg = seg_bufs(nullptr, 0, 0, 0);
    STK_HIP(launch_emit(e, out_mass != nullptr, st));
    STK_HIP(launch_dftopk_tail(status, out_p, n, out_mass, plan.g_emit, st));
    return SOFT_TOPK_OK;
}

size_t soft_topk_rows_workspace_bytes(int64_t rows, int64_t n_row)
{
    (void)rows;
    (void)n_row;
    return 0;  // every row length runs in the batched kernels, in registers or streamed
}

int soft_topk_rows_forward(const float* scores, int64_t rows, int64_t n_row, double k, double alpha, float* out_p,
                           double* out_b, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!scores || !out_p || !out_b || !rows_ok(rows, n_row))
        return SOFT_TOPK_EINVAL;
    if (!(alpha > 0.0) || !isfinite(alpha) || !(k > 0.0) || !(k < (double)n_row) || !isfinite(k))
        return SOFT_TOPK_EINVAL;
    (void)workspace;
    (void)workspace_bytes;
    RowsArgs a = rows_args(scores, rows, n_row, alpha);
    a.p = out_p;
    a.b = out_b;
    a.k = k;
    STK_HIP(launch_rows(a, true, static_cast<hipStream_t>(stream)));
    return SOFT_TOPK_OK;
}

int soft_topk_rows_backward(const float* grad_p, const float* scores, int64_t rows, int64_t n_row, double alpha,
                            const double* b, float* grad_s, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!grad_p || !scores || !b || !grad_s || !rows_ok(rows, n_row))
        return SOFT_TOPK_EINVAL;
    if (!(alpha > 0.0) || !isfinite(alpha))
        return SOFT_TOPK_EINVAL;
    (void)workspace;
    (void)workspace_bytes;
    RowsArgs a = rows_args(scores, rows, n_row, alpha);
    a.g = grad_p;
    a.grad = grad_s;
    a.b_in = b;
    STK_HIP(launch_rows(a, false, static_cast<hipStream_t>(stream)));
    return SOFT_TOPK_OK;
}

int soft_topk_debug_sample(const float* scores, int64_t n, double alpha, uint64_t seed, int32_t m,
                           float* out_samples, void* stream)
{
    if (!scores || !out_samples || !n_ok(n) || m < 1 || m > (1 << 24) || !(alpha > 0.0) || !isfinite(alpha))
        return SOFT_TOPK_EINVAL;
    STK_HIP(launch_debug_sample(scores, n, (float)alpha, seed, m, out_samples, static_cast<hipStream_t>(stream)));
    return SOFT_TOPK_OK;
}

}  // extern "C"
