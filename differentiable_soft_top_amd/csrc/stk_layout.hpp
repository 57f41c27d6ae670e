// stk_layout.hpp -- device status block, per-work-group partials, workspace
// plan and the host launchers of every kernel of the soft top-k path.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace stk {

// ---- fixed launch shapes -------------------------------------------------
constexpr int kStreamThreads = 256;      // streaming kernels (pass-1, emit, VJP)
// Streaming kernels walk tiles in grid-stride order; their grids are capped
// at these work-group counts (measured on MI355X: a few resident work-groups
// per CU sweeping the vectors together stream fastest).  Emission and VJP
// tiles hold kB float4 per lane: the larger batch from kStreamLargeMin
// scores on, the smaller one below (more work-groups for short vectors).
constexpr int kPass1Threads = 256;       // pass-1 work-group
constexpr int kPass1TileScores = 16 * kPass1Threads;  // scores per pass-1 tile (16 per lane)
constexpr int kEmitBatchLarge = 8;
constexpr int kEmitBatchSmall = 2;
constexpr int kVjpBatchLarge = 4;
constexpr int kVjpBatchSmall = 1;
constexpr int64_t kStreamLargeMin = 1 << 24;
constexpr int kGridPass1 = 2048;
constexpr int kPass1TilesPerGroup = 5;
constexpr int kCUs = 256;                // compute units of an MI355X
constexpr int kGridEmit = 8192;           // measured at 1e8: 142 us against 150 at 2048
// VJP grids: vectors past kStreamLargeMin stream from HBM, where fewer
// concurrent streams keep more DRAM pages open; smaller ones largely sit in
// the last-level cache and want more work-groups in flight.
constexpr int kGridVjpLarge = 256;
constexpr int kGridVjpSmall = 1024;
// The VJP over saturated-score segments is bound by dependent round trips,
// not by DRAM pages: it wants several work-groups per CU.
constexpr int kGridVjpSegReduce = 1024;
constexpr int kGridVjpSegApply = 1024;
constexpr int kSelectThreads = 1024;     // bracket select
constexpr int kSolveThreads = 512;       // segment solve
constexpr int kCandCap = 32768;          // candidate keys the select step holds (32 per thread)
constexpr int kFilterPer = 1024;         // samples per filter work-group (one per thread)
// Saturated-score segments.  A segment is one wave's share of a large VJP
// tile: 1024 scores, lane l holding value i (0..15) at float4 (tile * 1024 +
// (i / 4) * 256 + wave * 64 + l), component i % 4 (the emission walks the
// same tiles when it records them).  The emission, which knows b, marks
// in each segment the scores whose fp32 density d_i is not 0; a segment with
// at most kSegCap of them ("listed") keeps their d values.  The VJP then
// takes d from there instead of recomputing it from the scores: zero for
// every other score, which is what the scores give.  Used from kSegMinN
// scores on.
constexpr int kSegScores = 1024;
constexpr int kSegCap = 256;
constexpr uint32_t kSegDense = 0xFFFFFFFFu;
constexpr int64_t kSegMinN = 1 << 22;  // measured: from 10^7 scores on the record pays
static_assert(kStreamThreads == 256 && kVjpBatchLarge == 4,
              "segment geometry: large VJP tiles of 256 x 4 float4");
constexpr int kRowMax = 8192;            // longest row held in one work-group's registers (single vectors, sorted; rows' backward)
constexpr int kRefineRowMax = 2048;      // longest row the batched forward refines in a lane group
constexpr int kBuckets = 512;            // value buckets of the band sort
constexpr int kBucketCap = 8192;         // largest group the solve sorts in LDS
// The band is sorted whole (no buckets) when its expected size, n times the
// bracket's sample-rank width over m, is at most this.  With the bracket's
// ends at +-z binomial standard deviations, the band count spreads by about
// sqrt(2)/(2z) of that expectation (0.14 at z = 5), so the cut-off sits over
// four spreads below kBucketCap; a band that outgrows the sort anyway is
// bucketed afterwards, without a new pass.
constexpr double kDirectPredictMax = 5120.0;
constexpr int kBandGroups = 128;         // work-groups of band histogram/scatter
constexpr int kBandChunkMin = 2048;      // band elements per such work-group (at least)
constexpr int kSortThreads = 256;        // threads of bucket-sort / tile work-groups
constexpr int kTile = 4096;              // sorted elements per group in the full-sort solve
constexpr int kRadixThreads = 256;
constexpr int kRadixKeysPerThread = 32;
constexpr int kRadixTile = kRadixThreads * kRadixKeysPerThread;  // 8192 keys
constexpr int kRadixBins = 256;
// The per-tile digit counts ([tile][digit], one 1 KiB row per tile) are
// scanned in chunks of tiles: at most kRadixMaxChunks chunks, each of at
// least kRadixMinChunk tiles.
constexpr int kRadixMinChunk = 16;
constexpr int kRadixMaxChunks = 128;
__host__ __device__ constexpr int32_t radix_chunk_tiles(int32_t g)
{
    return (g + kRadixMaxChunks - 1) / kRadixMaxChunks > kRadixMinChunk ? (g + kRadixMaxChunks - 1) / kRadixMaxChunks
                                                                        : kRadixMinChunk;
}
constexpr int64_t kNontemporalMin = 1 << 25;  // outputs of at least 128 MiB bypass the caches
// Partition refinement of the band (no sort): one work-group holds up to
// kIterOneCap band values in LDS and runs at most kIterOneMax passes;
// larger bands (and all scores after a band overflow) take a chain of step
// kernels of kIterGroups work-groups.  The band goes to one work-group when
// its expected size is at most kIterOnePredictMax (about four binomial
// spreads below the cap, as for the whole-band sort).
constexpr int kIterOneThreads = 256;      // 4 waves: reductions cost per wave, the passes do not
constexpr int kIterOnePer = 64;
constexpr int kIterOneCap = kIterOneThreads * kIterOnePer;
constexpr int kIterOneMax = 16;
constexpr double kIterOnePredictMax = 10240.0;
constexpr int kIterThreads = 256;
constexpr int kIterGroups = 256;
constexpr int kIterGroupsAll = 1024;     // step grid known to refine every score (4 waves per SIMD for its fp64 terms)
constexpr int kIterStepsMin = 2;         // step kernels of a chain: the recent calls' passes, within these
constexpr int kIterStepsMax = 8;
constexpr int kIterPassesMax = 16;       // passes over all chains of one round before the band is sorted

// ---- solve status codes (Status::solve_state) ----------------------------
enum SolveState : uint32_t {
    kSolveNotRun = 0,
    kSolveOk = 1,
    kSolveRejectLow = 2,       // M(a_L) < k: b below the bracket
    kSolveRejectHigh = 3,      // M(a_R) > k: b at/above the bracket
    kSolveOverflow = 4,        // band did not fit its buffer
    kSolveNonfinite = 5,
    kSolveBucketOverflow = 6,  // a band bucket exceeded the LDS sort capacity
    kSolveDirectOverflow = 7,  // the band exceeded the whole-band sort (bucket it instead)
    kSolveIterLimit = 8,       // partition refinement did not end within its passes
    kSolveIterBig = 9,         // the band exceeded the one-work-group refinement
    kSolveIterMore = 10,       // the step kernels ran out before the end (resume the chain)
};

// Device status block at workspace offset 0.  Every field is written by a
// kernel; the host reads the whole block back once per forward round.
struct alignas(16) Status {
    // bracket (select step)
    float aL, aR;
    uint32_t select_info;        // bit0 candidate overflow, bit1 / bit2 left / right end conservative
    uint32_t cand_count;         // candidates over all filter work-groups
    uint32_t lo_key, hi_key;     // keys where every group's candidates overlap: ranks exact in between
    uint32_t below_n;            // samples below their group's lower bound
    uint32_t pad0;
    // pass-1 totals
    double SL, SR;               // sum_{s<a_L} e^{(s-a_L)/alpha}, sum_{s>=a_R} e^{-(s-a_R)/alpha}
    uint64_t nL, nR;             // tail counts
    uint64_t nB;                 // band count (global append cursor during pass-1)
    float bmin, bmax;            // range of the band values
    float smin, smax;            // range of all scores
    uint32_t nonfinite;
    uint32_t pad1;
    // segment solve
    double b;
    double massL, massR;         // M(a_L), M(a_R)
    uint32_t solve_state;
    uint32_t pad2;
    // certification pass (emit)
    double mass;                 // fp64 sum of p over all n
    uint32_t emit_done;
    uint32_t pad3;
    // saturated-score segments recorded by this forward's emission (cleared by
    // the select kernel and the full-sort reset), and what they were taken
    // from: the VJP uses them only for the same scores, n and alpha (and b)
    uint32_t seg_valid;
    uint64_t seg_n;
    double seg_alpha;
    uint64_t seg_scores;
    // the most frequent of a few candidate values in the band buffer, and
    // its estimated count there (band_mode_pick_kernel, after a band overflow)
    float tie_value;
    uint32_t tie_count;
    // the left tail of the split's first round (bracket [T+, a_R)), kept for
    // the closed form between the tied value T and the next float T+
    double tie_SL;
    uint64_t tie_nL;
    // partition refinement: what it refined (0: the band with the pass-1
    // tails, 1: every score) and the passes it took
    uint32_t iter_mode;
    uint32_t iter_steps;
};
static_assert(sizeof(Status) <= 256, "status block must fit 256 bytes");
static_assert(sizeof(Status) % 4 == 0, "status block is copied as 32-bit words");

// A host-visible mirror of the status block (pinned, fine-grained host
// memory) and the sequence number of the publication that filled it.
struct alignas(16) Mirror {
    Status st;
    uint32_t seq;
    uint32_t pad[3];
};

// Copy the status block to its host-visible mirror: one wave, one 32-bit
// word per lane.  The caller has synchronised the work-group, so every
// field this work-group wrote is in place.  The copy is released at system
// scope before seq is written, so a host that reads seq (with acquire) sees
// the whole block; without seq (0) the stores are complete when the kernel
// is.
__device__ __forceinline__ void publish_status(const Status* st, Mirror* mirror, uint32_t seq)
{
    constexpr int kWords = (int)(sizeof(Status) / 4);
    static_assert(kWords <= 64, "one word per lane of one wave");
    if (mirror == nullptr || threadIdx.x >= 64)
        return;
    if ((int)threadIdx.x < kWords)
        reinterpret_cast<volatile uint32_t*>(&mirror->st)[threadIdx.x] =
            reinterpret_cast<const volatile uint32_t*>(st)[threadIdx.x];
    if (seq != 0u) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");  // system scope, release only
        if (threadIdx.x == 0)
            *reinterpret_cast<volatile uint32_t*>(&mirror->seq) = seq;
    }
}

struct alignas(16) Pass1Partial {
    double SL, SR;
    uint64_t nL, nR;
    float bmin, bmax, smin, smax;
    uint32_t nonfinite;
    uint32_t pad[3];
};

// Summary of one sorted group (a band bucket or a tile of the full sort):
// count, first and last value, start offset in the sorted array,
// TA = sum e^{(x - hi)/alpha}, TB = sum e^{-(x - lo)/alpha}.
struct alignas(16) GroupAgg {
    double TA, TB;
    float lo, hi;
    uint32_t cnt;
    uint32_t start;
};

// Per-group scan results of the segment solve: prefix sum anchored at the
// group's last value (Pv), suffix of everything after the group anchored at
// its first point (Sx, Sv; Sx = +inf when empty) and the count of scores
// after the group (Cafter).
struct alignas(16) GroupScan {
    double Pv;
    double Sx;
    double Sv;
    uint64_t Cafter;
};

// ---- workspace plan --------------------------------------------------------
struct Plan {
    int64_t n;
    int32_t m;                   // samples
    int64_t cap;                 // band capacity
    int32_t g_pass1;             // work-groups of pass-1 (and of the range pass)
    int32_t g_emit;              // work-groups of the emission
    int32_t g_band;              // max work-groups of band histogram/scatter
    int32_t n_tiles;             // groups of the full-sort solve
    int32_t g_radix;             // radix tiles
    size_t off_status, off_samples, off_frec, off_p1part, off_band, off_band_sorted;
    size_t off_hist, off_bstart, off_agg, off_scan, off_emitpart, off_iter, off_keys0, off_keys1, off_rhist, off_super;
    int64_t n_seg;               // saturated-score segments (0: not used at this n)
    size_t off_seg_cnt, off_seg_ent;
    size_t total;
};

Plan make_plan(int64_t n, int32_t m, int64_t cap);

// ---- host launchers (each enqueues on `stream`, returns the launch status) --
// What one filter work-group reports: its samples below its lower bound,
// its candidates (stored in its own region of kFilterPer keys) and the
// bounds themselves (0 / all-ones when open).
struct alignas(16) FilterRec {
    uint32_t below, cand, lo, hi;
};

struct SampleArgs {
    const float* s;
    int64_t n;
    float alpha;
    uint32_t k0, k1;              // Philox key (seed low / high word)
    int32_t m;                    // samples
    int64_t r_left, r_right;      // 1-based target ranks (0 = -inf, m+1 = +inf)
    double q;                     // target quantile 1 - k/n
    uint32_t* cand;               // [groups * kFilterPer] candidate keys, one region per group
    FilterRec* rec;               // [groups]
};

struct SelectArgs {
    const uint32_t* cand;
    const FilterRec* rec;
    int32_t groups;               // filter work-groups, ceil(m / kFilterPer)
    int32_t m;
    int64_t r_left, r_right;
    Status* st;
};

hipError_t launch_localize(const SampleArgs& sa, const SelectArgs& se, hipStream_t stream);
// After a band or bucket overflow: estimate, from a sample of the band
// buffer (its first min(nB, cap) entries), the count of the most frequent
// of eight candidate values taken from it (Status::tie_value, tie_count).
// `counts`: scratch for 64 x 8 u32 per-chunk candidate counts.
hipError_t launch_band_mode(const float* band, int64_t cap, Status* st, uint32_t* counts, hipStream_t stream);
// Start a round on an explicit bracket [aL, aR) (instead of the sampler's):
// the bracket and the per-round fields the select kernel would set.
hipError_t launch_set_bracket(Status* st, float aL, float aR, bool keep_left_tail, hipStream_t stream);
// Hand a root found on the host to the emission: b into out_b and the
// status, and the solve state OK.
// b strictly between the tied value T and T+ (see tie_root_kernel); the
// status is published to `mirror` with `seq` either way.
struct TieRootArgs {
    Status* st;
    double* out_b;
    int64_t n;
    double k, alpha, log2e_over_alpha;
    Mirror* mirror;
    uint32_t seq;
};
hipError_t launch_tie_root(const TieRootArgs& a, hipStream_t stream);
hipError_t launch_debug_sample(const float* s, int64_t n, float alpha, uint64_t seed, int32_t m,
                               float* out_samples, hipStream_t stream);

// Saturated-score segment storage (all null when not used).
struct SegBufs {
    uint32_t* cnt;                // [n_seg] listed count, or kSegDense
    uint64_t* ent;                // [n_seg][kSegCap] listed entries in (value index, lane) order:
                                  // fp32 density d (low word), place in the segment (high word)
};

struct Pass1Args {
    const float* s;
    int64_t n;
    double log2e_over_alpha;
    float* band;
    int64_t cap;
    Pass1Partial* partials;
    int32_t blocks;
    int32_t count_only;           // keep no band: only count it (a band expected to overflow)
    Status* st;
};
hipError_t launch_pass1(const Pass1Args& a, hipStream_t stream);
hipError_t launch_pass1_finalize(const Pass1Partial* partials, int blocks, Status* st, hipStream_t stream);
hipError_t launch_range(const float* s, int64_t n, Pass1Partial* partials, int blocks, hipStream_t stream);

struct BandArgs {
    const Pass1Partial* p1;       // pass-1 partials (band range when the bracket is open-ended)
    int32_t p1_blocks;
    Pass1Partial* p1_super;       // [kBuckets] partials folded by groups of p1_blocks/kBuckets
    const float* band;
    float* band_sorted;
    int64_t cap;
    uint32_t* hist;               // [g_band][kBuckets]
    uint32_t* bstart;             // [kBuckets + 1]
    GroupAgg* agg;                // [kBuckets]
    int32_t blocks;               // g_band
    double log2e_over_alpha;
    Status* st;
};
hipError_t launch_band_sort(const BandArgs& a, hipStream_t stream);

struct SolveArgs {
    const Pass1Partial* p1;       // pass-1 partials (tails of the bracketed route)
    int32_t p1_blocks;
    const Pass1Partial* p1_super; // the same folded to kBuckets entries by the band sort
    const float* sorted;          // sorted values
    const GroupAgg* agg;
    GroupScan* scan;              // scratch [groups]
    int32_t groups;
    int32_t tails;                // 1: bracketed (tails from status), 0: full sort (no tails)
    int32_t direct;               // bracketed: 1 = sort the unbucketed band (at `sorted`) whole
    int64_t cap;                  // band capacity (bracketed route)
    double k;
    double alpha;
    double log2e_over_alpha;
    double* out_b;
    Status* st;
    Mirror* mirror;               // host-visible copy of the status written at the end (may be null)
    uint32_t seq;                 // its publication number (0: none)
};
hipError_t launch_solve(const SolveArgs& a, hipStream_t stream);

// Partition sums of one work-group at a split point r: the sum of
// e^{-(s - r)/alpha} over its scores above r (A), of e^{(s - r)/alpha} over
// the others (B), the count above r (N), and the nearest scores on each side.
struct alignas(16) SplitPartial {
    double A, B;
    uint64_t N;
    float lo, hi;
};

// State of the step kernels between launches (workspace): the split points
// of the last two steps (alternate steps use alternate entries, so no
// work-group reads what another work-group of the same step writes), where
// a chain that ran out stopped, and whether the refinement has ended.
struct alignas(16) IterState {
    double x[2];                  // split points of alternate steps
    double resume_x;              // where a chain that ran out stopped
    uint32_t done;
    uint32_t pad;
};

struct IterArgs {
    const float* band;            // the unsorted band of the round (st->nB values)
    int64_t cap;                  // its capacity: a larger band refines every score instead
    const float* s;               // all scores
    int64_t n;
    const Pass1Partial* p1;       // pass-1 partials (tails, band range, finiteness)
    int32_t p1_blocks;
    IterState* is;                // step kernels' state
    SplitPartial* part;           // [2][kIterGroupsAll] sums of alternate steps
    int32_t groups;               // work-groups of a step (kIterGroups, or kIterGroupsAll)
    int32_t passes_before;        // passes of earlier chains of this round (resumed)
    double k;
    double alpha;
    double log2e_over_alpha;
    double* out_b;
    Status* st;
    Mirror* mirror;               // host-visible status copy written at the end
    uint32_t seq;                 // its publication number
};
// One work-group (one_group), or a chain of `steps` step kernels and the
// final kernel (resume: start where the last chain stopped).
hipError_t launch_partition_solve(const IterArgs& a, bool one_group, int steps, bool resume, hipStream_t stream);

struct RadixArgs {
    const float* s;
    int64_t n;
    uint32_t* keys0;
    uint32_t* keys1;
    uint32_t* hist;               // [g_radix][kRadixBins] counts, then offsets; then [chunks][kRadixBins] chunk sums
    int32_t g_radix;
    uint32_t key_min;             // subtracted from every key
    int32_t passes;               // 8-bit digits to sort
    Status* st;
    uint32_t** sorted_out;        // receives keys0 or keys1 (host side)
};
hipError_t launch_radix_sort(const RadixArgs& a, hipStream_t stream);

struct TileArgs {
    uint32_t* keys;               // sorted keys (offset by key_min); overwritten with fp32 values
    int64_t n;
    uint32_t key_min;
    GroupAgg* agg;
    int32_t n_tiles;
    double log2e_over_alpha;
};
hipError_t launch_tile_aggregates(const TileArgs& a, hipStream_t stream);

struct EmitArgs {
    const float* s;
    int64_t n;
    double alpha;
    double log2e_over_alpha;
    const double* b;
    float* p;
    double* partials;
    int32_t blocks;
    Status* st;
    Mirror* mirror;               // host-visible copy of the status written by the mass fold (may be null)
    SegBufs seg;                  // used when pass-1 wrote them (st->seg_valid)
};
hipError_t launch_emit(const EmitArgs& a, bool fold_mass, hipStream_t stream);

struct VjpArgs {
    const float* g;
    const float* s;
    int64_t n;
    double alpha;
    double log2e_over_alpha;
    const double* b;
    float* grad;
    double* partials;             // [reduce_blocks][2]
    int32_t blocks;               // work-groups of the gradient kernel
    int32_t reduce_blocks;        // work-groups of the (D, G) reduction
    // the forward's saved segments (null: none); used only when its status
    // says they were taken from these scores, n, alpha and b
    const Status* fst;
    SegBufs seg;
    int64_t seg_tiles;            // large VJP tiles that have segments
    float* gl;                    // [n_seg][kSegCap] listed g values (backward workspace)
};
hipError_t launch_vjp(const VjpArgs& a, hipStream_t stream);

hipError_t launch_reset_status(Status* st, hipStream_t stream, bool open_bracket);

// Batched rows (rows x n_row, row-major, any n_row): lane groups, or one
// work-group per row (see launch_rows).
struct RowsArgs {
    const float* s;
    const float* g;               // backward: cotangent
    float* p;                     // forward: output
    float* grad;                  // backward: output
    double* b;                    // forward: per-row thresholds (output)
    const double* b_in;           // backward: per-row thresholds
    int64_t rows;
    int32_t n_row;
    double k, alpha, log2e_over_alpha;
    // the single-vector route (one row of more than 64 scores): the forward
    // kernel also folds the fp64 mass of its p into this status block and
    // publishes it (nullptr: no status)
    Status* st;
    Mirror* mirror;
    uint32_t seq;
};
hipError_t launch_rows(const RowsArgs& a, bool forward, hipStream_t stream);
// One row (rows == 1, n_row <= kRowMax) with the shortest chain per thread:
// the single-vector route, where latency matters rather than throughput.
hipError_t launch_row_alone(const RowsArgs& a, bool forward, hipStream_t stream);

// The threshold curve: every score in ascending order with the mass
// M(x_j) = sum_i F((s_i - x_j)/alpha) it would select as threshold, from the
// full-sort route's sorted values and tile summaries.
struct CurveArgs {
    const float* sorted;          // ascending values (the full sort's output)
    const GroupAgg* agg;          // [n_tiles] tile summaries
    void* ex;                     // [n_tiles] scratch: sums before / after each tile
    int64_t n;
    int32_t n_tiles;
    double log2e_over_alpha;
    float* out_sorted;
    double* out_mass;
};
hipError_t launch_curve(const CurveArgs& a, hipStream_t stream);

// A single vector of at most kRowMax scores solved by the row kernels: one
// work-group folds the fp64 sum of the emitted p, writes a fresh status
// block (b, mass, the non-finite flag; no segment record) and publishes it.
struct SingleArgs {
    const float* p;
    const double* b;
    int64_t n;
    Status* st;
    Mirror* mirror;
    uint32_t seq;
};
hipError_t launch_single_status(const SingleArgs& a, hipStream_t stream);

// DFTopK comparator: radix selection of the k-th and (k+1)-th largest
// scores (three passes of 11, 11 and 10 key bits), then b at their midpoint.
constexpr int kDftThreads = 512;
constexpr int kDftBins = 2048;                 // digits of the 11-bit passes
constexpr int kDftRowWords = 2 * kDftBins + 64;  // two targets' counts, the NaN count, padding
constexpr int kDftMaxGroups = 512;
constexpr int kDftTileScores = kDftThreads * 8 * 4;

// Before pass P: for the (k+1)-th largest (target 0) and the k-th largest
// (target 1), the key digits chosen so far and the rank left among the keys
// that carry them.
struct alignas(16) DftState {
    uint32_t prefix[2];
    uint32_t rank[2];
};

struct DftArgs {
    const float* s;
    int64_t n;
    int64_t k;
    uint32_t* rows;               // [groups][kDftRowWords] per-work-group counts
    uint32_t* totals;             // [3][kDftRowWords] per-pass totals
    DftState* state;              // [3] state before each pass
    int32_t groups;
    Status* st;                   // b, the NaN flag and the emission's mass
    double* out_b;
};
hipError_t launch_dftopk_threshold(const DftArgs& a, hipStream_t stream);
hipError_t launch_dftopk_tail(const Status* st, float* p, int64_t n, double* out_mass, int32_t blocks,
                              hipStream_t stream);

}  // namespace stk
