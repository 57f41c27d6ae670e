// sample_select.hip -- localisation step of the bracketed solver.
//
// gist.science summary of Fast LapSum, section 2.2, "Probabilistic
// Bracketing" step 1 (and the aiqbench.com abstract): a small sample of
// kernel-noised scores is drawn and two of its order statistics, whose ranks
// come from the binomial law, form a bracket [a_L, a_R) around b.
//
// Why the sample is kernel-noised: with I uniform on {0..n-1} and E a
// standard Laplace variable, Y = s_I + alpha*E satisfies
// P(Y > b) = (1/n) sum_i F((s_i - b)/alpha) = M(b)/n, so b is exactly the
// (1 - k/n)-quantile of Y, and the number of samples at or below b is
// Binomial(m, 1 - k/n) whatever the scores are.
#include "stk_common.hpp"
#include "stk_layout.hpp"
#include "stk_prof.hpp"
#include "stk_scan.hpp"

namespace stk {

// Sample j: counter (j, 0, 0, 0), key (seed lo, seed hi).  Words 0/1 give a
// 64-bit uniform u64; the index is the high half of u64 * n (unbiased to
// 2^-64 n, where a 32-bit product would skew indices by up to n/2^32).  Word 2
// gives u in (0,1) and E = F^{-1}(u).  Samples are regenerated wherever they
// are needed (same counter, same value), never stored.
__device__ __forceinline__ float sample_value(const float* __restrict__ s, int64_t n, float alpha, uint32_t k0,
                                              uint32_t k1, uint32_t j)
{
    const Philox4 r = philox4x32_10(j, 0u, 0u, 0u, k0, k1);
    const uint64_t u64 = ((uint64_t)r.v[1] << 32) | (uint64_t)r.v[0];
    const uint64_t idx = __umul64hi(u64, (uint64_t)n);  // < n
    const double u = ((double)r.v[2] + 0.5) * (1.0 / 4294967296.0);
    const double e = (u < 0.5) ? log(2.0 * u) : -log(2.0 * (1.0 - u));
    return (float)((double)s[idx] + (double)alpha * e);
}

// Diagnostic: write the m samples (soft_topk_debug_sample).
__global__ __launch_bounds__(256) void sample_kernel(const float* __restrict__ s, int64_t n, float alpha,
                                                     uint32_t k0, uint32_t k1, int32_t m,
                                                     float* __restrict__ out)
{
    const int32_t j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= m)
        return;
    out[j] = sample_value(s, n, alpha, k0, k1, (uint32_t)j);
}

hipError_t launch_debug_sample(const float* s, int64_t n, float alpha, uint64_t seed, int32_t m,
                               float* out_samples, hipStream_t stream)
{
    const int blocks = (m + 255) / 256;
    STK_LAUNCH(kKSample, stream, sample_kernel, dim3(blocks), dim3(256), 0, stream, s, n, alpha,
               (uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32), m, out_samples);
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// The localisation in two kernels, so no single work-group has to draw all
// m samples (a CU ingests only ~10 GB/s of freshly written data, and the
// Philox rounds of 65536 samples would keep one CU busy for tens of us):
//   filter (m / kFilterPer groups) -- each group draws its kFilterPer
//          samples, takes two of its own order statistics that enclose the
//          targets with a wide margin (expected local rank -+ 7 local
//          binomial standard deviations - 4), counts its samples below the
//          lower one and stores those between them, in a region of its own;
//   select (1 group) -- with L the largest group lower bound and H the
//          smallest upper bound, the rank of any x in [L, H] among all m
//          samples is (samples below their group's bound) + (candidates
//          <= x), so the target order statistics are the candidates of
//          ranks r - below; it also clears the per-round counters of the
//          status block (it runs right before pass-1).
// Order statistics are selected digit by digit (block_select2), not sorted.
// A target that falls outside [L, H] or outside the candidates (a margin
// broken, about 1e-9 per group and side) is replaced by a conservative
// bound (the smallest group lower bound / largest upper bound, or an open
// end): the bracket only widens and the certificate still decides.
// ---------------------------------------------------------------------------
namespace {

constexpr int kFilterThreads = kFilterPer;  // one sample per thread
static_assert(kCandCap == 32 * kSelectThreads, "select shapes cover the candidate capacity");

// Local rank bounds of a group of mw samples for global ranks (rl, rr) of
// m; -1 = open end.
__device__ __forceinline__ void local_ranks(int64_t rl, int64_t rr, int32_t m, int32_t mw, double q, int64_t* lo,
                                            int64_t* hi)
{
    const double sd = sqrt((double)mw * q * (1.0 - q));
    *lo = -1;
    *hi = -1;
    if (rl >= 1) {
        const double e = (double)mw * (double)rl / (double)m;
        const int64_t r = (int64_t)floor(e - 7.0 * sd - 4.0);
        *lo = r >= 1 ? r : -1;
    }
    if (rr <= (int64_t)m) {
        const double e = (double)mw * (double)rr / (double)m;
        const int64_t r = (int64_t)ceil(e + 7.0 * sd + 4.0);
        *hi = r <= (int64_t)mw ? r : -1;
    }
}

// The keys at ranks r0 / r1 of the cnt candidates spread over the group
// regions (start offsets off[0..groups], R per thread).
template <int R>
__device__ void select_from(const uint32_t* __restrict__ cand, const uint32_t* off, int groups, int cnt, int64_t r0,
                            int64_t r1, uint32_t* hist, uint32_t* state, uint32_t* out)
{
    uint32_t v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = threadIdx.x * R + r;
        uint32_t key = 0xFFFFFFFFu;
        if (i < cnt) {
            // the region holding candidate i: the last w with off[w] <= i
            int lo = 0, hi = groups;  // off[lo] <= i < off[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (off[mid] <= (uint32_t)i)
                    lo = mid;
                else
                    hi = mid;
            }
            key = cand[(size_t)lo * kFilterPer + (i - off[lo])];
        }
        v[r] = key;
    }
    block_select2<kSelectThreads, R>(v, cnt, r0, r1, hist, state, out);
}

}  // namespace

__global__ __launch_bounds__(kFilterThreads) void filter_kernel(SampleArgs a)
{
    constexpr int kWaves = kFilterThreads / kWave;
    __shared__ __align__(16) uint32_t hist[1024];  // block_select2 reads it as uint4
    __shared__ uint32_t sstate[4 + 2 * (1024 / kWave)];  // block_select2 state (1024 threads)
    __shared__ uint32_t bounds[2];
    __shared__ uint32_t wcnt[2][kWaves];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int32_t j0 = (int32_t)blockIdx.x * kFilterPer;
    const int32_t mw = a.m - j0 < kFilterPer ? a.m - j0 : kFilterPer;
    const bool valid = tid < mw;
    const uint32_t key = valid ? float_to_key(sample_value(a.s, a.n, a.alpha, a.k0, a.k1, (uint32_t)(j0 + tid)))
                               : 0xFFFFFFFFu;
    int64_t rlo, rhi;
    local_ranks(a.r_left, a.r_right, a.m, mw, a.q, &rlo, &rhi);
    if (tid == 0) {
        bounds[0] = 0u;           // open lower bound
        bounds[1] = 0xFFFFFFFFu;  // open upper bound
    }
    uint32_t v[1] = {key};
    block_select2<kFilterThreads, 1>(v, mw, rlo, rhi, hist, sstate, bounds);
    const uint32_t lo = bounds[0], hi = bounds[1];
    const bool below = valid && key < lo;
    const bool cand = valid && key >= lo && key <= hi;
    const uint64_t bm = __builtin_amdgcn_ballot_w64(below);
    const uint64_t cm = __builtin_amdgcn_ballot_w64(cand);
    if (lane == 0) {
        wcnt[0][wave] = (uint32_t)__popcll(bm);
        wcnt[1][wave] = (uint32_t)__popcll(cm);
    }
    __syncthreads();
    uint32_t woff = 0, tot_c = 0, tot_b = 0;
    for (int w = 0; w < kWaves; ++w) {
        woff += w < wave ? wcnt[1][w] : 0u;
        tot_c += wcnt[1][w];
        tot_b += wcnt[0][w];
    }
    if (cand)
        a.cand[(size_t)blockIdx.x * kFilterPer + woff + rank_in_mask(cm)] = key;
    if (tid == 0) {
        FilterRec r;
        r.below = tot_b;
        r.cand = tot_c;
        r.lo = lo;
        r.hi = hi;
        a.rec[blockIdx.x] = r;
    }
}

__global__ __launch_bounds__(kSelectThreads) void select_kernel(SelectArgs se)
{
    constexpr int kWaves = kSelectThreads / kWave;
    static_assert(kSelectThreads == 1024 && kFilterThreads == 1024, "select state sized for 1024 threads; one thread per filter group (m <= 262144)");
    __shared__ __align__(16) uint32_t hist[1024];  // block_select2 reads it as uint4
    __shared__ uint32_t sstate[4 + 2 * (1024 / kWave)];  // block_select2 state (1024 threads)
    __shared__ uint32_t sel[2];
    __shared__ uint32_t off[kSelectThreads + 1];
    __shared__ uint32_t wred[5][kWaves];
    Status* st = se.st;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int G = se.groups;

    // ---- the groups' records: candidate offsets, totals, bound extremes ------
    FilterRec r;
    r.below = 0;
    r.cand = 0;
    r.lo = 0u;           // neutral for the max of lower bounds
    r.hi = 0xFFFFFFFFu;  // neutral for the min of upper bounds
    uint32_t lo_min = 0xFFFFFFFFu, hi_max = 0u;
    if (tid < G) {
        r = se.rec[tid];
        lo_min = r.lo;
        hi_max = r.hi;
    }
    uint32_t incl = r.cand;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o, kWave);
        if (lane >= o)
            incl += t;
    }
    uint32_t bsum = r.below, lmax = r.lo, hmin = r.hi, lmin = lo_min, hmax = hi_max;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        bsum += __shfl_xor(bsum, o, kWave);
        lmax = max(lmax, (uint32_t)__shfl_xor(lmax, o, kWave));
        hmin = min(hmin, (uint32_t)__shfl_xor(hmin, o, kWave));
        lmin = min(lmin, (uint32_t)__shfl_xor(lmin, o, kWave));
        hmax = max(hmax, (uint32_t)__shfl_xor(hmax, o, kWave));
    }
    if (lane == kWave - 1)
        wred[0][wave] = incl;  // wave total of candidates
    if (lane == 0) {
        wred[1][wave] = bsum;
        wred[2][wave] = lmax;
        wred[3][wave] = hmin;
        wred[4][wave] = lmin;
    }
    __syncthreads();
    uint32_t base = 0, C = 0, B = 0, L = 0u, H = 0xFFFFFFFFu, Lmin = 0xFFFFFFFFu;
    for (int w = 0; w < kWaves; ++w) {
        base += w < wave ? wred[0][w] : 0u;
        C += wred[0][w];
        B += wred[1][w];
        L = max(L, wred[2][w]);
        H = min(H, wred[3][w]);
        Lmin = min(Lmin, wred[4][w]);
    }
    __syncthreads();
    if (lane == 0)
        wred[4][wave] = hmax;
    if (tid <= G)
        off[tid] = base + incl - r.cand;  // exclusive prefix; off[G] = C
    if (tid == 0)
        off[G] = C;
    __syncthreads();
    uint32_t Hmax = 0u;
    for (int w = 0; w < kWaves; ++w)
        Hmax = max(Hmax, wred[4][w]);

    // ---- the target order statistics among the candidates --------------------
    const int64_t rl = se.r_left, rr = se.r_right;
    const bool overflow = C > (uint32_t)kCandCap;
    const bool left_open = rl <= 0;
    const bool right_open = rr > (int64_t)se.m;
    const int64_t r0 = rl - (int64_t)B, r1 = rr - (int64_t)B;
    const bool left_in = !left_open && !overflow && r0 >= 1 && r0 <= (int64_t)C;
    const bool right_in = !right_open && !overflow && r1 >= 1 && r1 <= (int64_t)C;
    if (tid == 0) {
        sel[0] = 0u;
        sel[1] = 0xFFFFFFFFu;
    }
    if (left_in || right_in) {
        // the shape follows the candidate count (uniform branch)
        const int cnt = (int)C;
        const int64_t s0 = left_in ? r0 : -1, s1 = right_in ? r1 : -1;
        if (cnt <= kSelectThreads)
            select_from<1>(se.cand, off, G, cnt, s0, s1, hist, sstate, sel);
        else if (cnt <= 2 * kSelectThreads)
            select_from<2>(se.cand, off, G, cnt, s0, s1, hist, sstate, sel);
        else if (cnt <= 4 * kSelectThreads)
            select_from<4>(se.cand, off, G, cnt, s0, s1, hist, sstate, sel);
        else if (cnt <= 8 * kSelectThreads)
            select_from<8>(se.cand, off, G, cnt, s0, s1, hist, sstate, sel);
        else if (cnt <= 16 * kSelectThreads)
            select_from<16>(se.cand, off, G, cnt, s0, s1, hist, sstate, sel);
        else
            select_from<32>(se.cand, off, G, cnt, s0, s1, hist, sstate, sel);
    }
    if (tid == 0) {
        uint32_t info = overflow ? 1u : 0u;
        float aL, aR;
        if (left_open) {
            aL = -INFINITY;
        } else if (left_in && sel[0] >= L && sel[0] <= H) {
            aL = key_to_float(sel[0]);
        } else {
            // conservative: no group's lower bound exceeds the target w.h.p.
            aL = Lmin == 0u ? -INFINITY : key_to_float(Lmin);
            info |= 2u;
        }
        if (right_open) {
            aR = INFINITY;
        } else if (right_in && sel[1] >= L && sel[1] <= H) {
            aR = key_to_float(sel[1]);
        } else {
            aR = Hmax == 0xFFFFFFFFu ? INFINITY : key_to_float(Hmax);
            info |= 4u;
        }
        st->aL = aL;
        st->aR = aR;
        st->select_info = info;
        st->cand_count = C;
        st->lo_key = L;
        st->hi_key = H;
        st->below_n = B;
        // per-round counters of the passes that follow
        st->nB = 0;
        st->solve_state = kSolveNotRun;
        st->emit_done = 0;
        st->nonfinite = 0;
        st->seg_valid = 0;
    }
}

// ---------------------------------------------------------------------------
// A heavily repeated value in the band (a cluster of exact ties, such as
// many scores at one quantised level) makes the band overflow however the
// bracket is drawn: no bracket around b can leave the tied scores out when
// b lies among them.  The host then splits the bracket at that value, which
// puts the whole cluster into one tail.  These kernels find the candidate:
// eight values taken from evenly spread places in the band buffer, each
// counted over kModeChunks contiguous runs of up to kModeRun entries spread
// evenly over the buffer (65,536 entries in all, read coalesced by
// kModeChunks work-groups), then folded by one small work-group.  Only a
// heuristic for the next bracket: the certificate of that round decides.
// ---------------------------------------------------------------------------
constexpr int kModeThreads = 256;
constexpr int kModeCands = 8;
constexpr int kModeChunks = 64;
constexpr int kModeRun = 1024;  // entries per chunk (4 per thread)

__device__ __forceinline__ int64_t mode_band_len(const Status* st, int64_t cap)
{
    return (int64_t)st->nB < cap ? (int64_t)st->nB : cap;
}

// [start, end) of chunk j of a band of m entries
__device__ __forceinline__ void mode_chunk(int64_t m, int j, int64_t* start, int64_t* end)
{
    const int64_t s = (int64_t)j * m / kModeChunks;
    const int64_t e = (int64_t)(j + 1) * m / kModeChunks;
    *start = s;
    *end = e - s < kModeRun ? e : s + kModeRun;
}

__device__ __forceinline__ float mode_cand(const float* band, int64_t m, int c)
{
    return band[(2 * c + 1) * m / (2 * kModeCands)];
}

__global__ __launch_bounds__(kModeThreads) void band_mode_count_kernel(const float* band, int64_t cap, const Status* st,
                                                                      uint32_t* counts)
{
    __shared__ uint32_t cnt[kModeThreads / kWave][kModeCands];
    const int tid = threadIdx.x;
    const int64_t m = mode_band_len(st, cap);
    int64_t start, end;
    mode_chunk(m, blockIdx.x, &start, &end);
    float cand[kModeCands];
    uint32_t my[kModeCands];
#pragma unroll
    for (int c = 0; c < kModeCands; ++c) {
        cand[c] = m > 0 ? mode_cand(band, m, c) : 0.0f;
        my[c] = 0u;
    }
    for (int64_t j = start + tid; j < end; j += kModeThreads) {
        const float v = band[j];
#pragma unroll
        for (int c = 0; c < kModeCands; ++c)
            my[c] += v == cand[c] ? 1u : 0u;
    }
#pragma unroll
    for (int c = 0; c < kModeCands; ++c) {
        const uint32_t w = wave_sum_u32(my[c]);
        if (lane_id() == 0)
            cnt[tid / kWave][c] = w;
    }
    __syncthreads();
    if (tid < kModeCands) {
        uint32_t t = 0u;
        for (int w = 0; w < kModeThreads / kWave; ++w)
            t += cnt[w][tid];
        counts[blockIdx.x * kModeCands + tid] = t;
    }
}

__global__ __launch_bounds__(kWave) void band_mode_pick_kernel(const float* band, int64_t cap, Status* st,
                                                              const uint32_t* counts)
{
    __shared__ uint32_t tot[kModeCands];
    const int tid = threadIdx.x;
    const int64_t m = mode_band_len(st, cap);
    if (tid < kModeCands) {
        uint32_t t = 0u;
        for (int j = 0; j < kModeChunks; ++j)
            t += counts[j * kModeCands + tid];
        tot[tid] = t;
    }
    __syncthreads();
    if (tid == 0) {
        int64_t S = 0;
        for (int j = 0; j < kModeChunks; ++j) {
            int64_t s, e;
            mode_chunk(m, j, &s, &e);
            S += e - s;
        }
        uint32_t best = 0u;
        float bv = 0.0f;
        for (int c = 0; c < kModeCands; ++c) {
            if (tot[c] > best) {
                best = tot[c];
                bv = mode_cand(band, m, c);
            }
        }
        st->tie_value = bv;
        st->tie_count = S > 0 ? (uint32_t)((double)best * (double)m / (double)S) : 0u;
    }
}

hipError_t launch_band_mode(const float* band, int64_t cap, Status* st, uint32_t* counts, hipStream_t stream)
{
    band_mode_count_kernel<<<kModeChunks, kModeThreads, 0, stream>>>(band, cap, st, counts);
    band_mode_pick_kernel<<<1, kWave, 0, stream>>>(band, cap, st, counts);
    return hipGetLastError();
}

__global__ void set_bracket_kernel(Status* st, float aL, float aR, int keep_left_tail)
{
    if (threadIdx.x == 0) {
        if (keep_left_tail) {
            st->tie_SL = st->SL;
            st->tie_nL = st->nL;
        }
        st->aL = aL;
        st->aR = aR;
        st->select_info = 0u;
        st->cand_count = 0u;
        st->lo_key = 0u;
        st->hi_key = 0u;
        st->below_n = 0u;
        st->nB = 0;
        st->solve_state = kSolveNotRun;
        st->emit_done = 0;
        st->nonfinite = 0;
        st->seg_valid = 0;
    }
}

hipError_t launch_set_bracket(Status* st, float aL, float aR, bool keep_left_tail, hipStream_t stream)
{
    set_bracket_kernel<<<1, kWave, 0, stream>>>(st, aL, aR, keep_left_tail ? 1 : 0);
    return hipGetLastError();
}

// The split at a tied value T put the cluster into the left tail of the
// round on [T+, a_R) (T+ the next float above T) and into the right tail of
// the round on [a_L, T).  When the first rejected low (M(T+) < k) and the
// second high (M(T) > k), b lies strictly between T and T+, inside the gap
// right of T.  The closed form of the full-sort solver (gist.science summary
// of Fast LapSum, section 2.2) there, with both sums anchored at T:
//   A = the left sum over every score <= T: the first round's left tail,
//       moved from its anchor T+ to T;
//   C = the count of scores > T: n less the first round's left count;
//   B = the right sum over the scores > T: the second round's right tail
//       (anchored at T) less the cluster, whose terms are exactly 1 each and
//       number nR - C.
// A root outside [T, T+] (which rounding alone could cause) leaves the
// round rejected, and the full sort decides.
__global__ void tie_root_kernel(TieRootArgs a)
{
    Status* st = a.st;
    if (threadIdx.x == 0) {
        const float T = st->tie_value;
        const float Tp = nextafterf(T, INFINITY);
        const double A = st->tie_SL * exp2(((double)Tp - (double)T) * a.log2e_over_alpha);
        const double C = (double)a.n - (double)st->tie_nL;
        const double B = st->SR - ((double)st->nR - C);
        bool ok = A > 0.0 && B > 0.0;
        double b = 0.0;
        if (ok) {
            b = gap_root(node(T, A), node(T, B), C, a.k, a.alpha, a.log2e_over_alpha);
            ok = b >= (double)T && b <= (double)Tp;
        }
        if (ok) {
            st->b = b;
            *a.out_b = b;
            st->solve_state = kSolveOk;
        }
    }
    __syncthreads();
    publish_status(st, a.mirror, a.seq);
}

hipError_t launch_tie_root(const TieRootArgs& a, hipStream_t stream)
{
    tie_root_kernel<<<1, kWave, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_localize(const SampleArgs& sa, const SelectArgs& se, hipStream_t stream)
{
    STK_LAUNCH(kKFilter, stream, filter_kernel, dim3(se.groups), dim3(kFilterThreads), 0, stream, sa);
    STK_LAUNCH(kKSelect, stream, select_kernel, dim3(1), dim3(kSelectThreads), 0, stream, se);
    return hipGetLastError();
}

}  // namespace stk
