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
// The localisation in two kernels, so no single work-group has to read all
// m samples (one CU ingests only ~10 GB/s of freshly written data):
//   pilot  (1 work-group)  -- the first P = min(m, kPilot) samples, two of
//          their order statistics that enclose the target ranks with a wide
//          margin (ranks from the host);
//   filter (m/1024 groups) -- every sample regenerated, counted if below the
//          lower pilot bound, appended to a candidate list if between them;
//   select (the last filter work-group to finish) -- the target order
//          statistics among the candidates, offset by the count below.
// Order statistics are read off a work-group sort of the keys held in
// registers (block_bitonic_regs).  If the candidates overflow or a target
// falls outside them, a pilot value with a more conservative rank is used
// (the bracket only widens, so the certificate still decides).  The pilot
// kernel also clears the per-round counters of the status block: it runs
// first in every bracketed round.
// ---------------------------------------------------------------------------
namespace {

// Sorting shapes: a full 1024-thread work-group (four waves per SIMD hide
// the latency of the dependent compare-exchange chains), as few keys per
// thread as the count allows.
constexpr int kPilotThreads = 1024;
constexpr int kPilotPer = kPilot / kPilotThreads;  // pilot keys per thread
static_assert(kPilot % kPilotThreads == 0, "pilot keys per thread");
static_assert(kCandCap == 16 * kSelectThreads, "select shapes cover the candidate capacity");

// The keys at 1-based ranks r0 and r1 of the sorted blocked registers v
// (kThreads * R positions) go to out[0] / out[1] (a rank outside the
// positions writes nothing).
template <int R>
__device__ __forceinline__ void pick_ranks(const uint32_t (&v)[R], int64_t r0, int64_t r1, uint32_t* out)
{
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t rank = (int64_t)threadIdx.x * R + r + 1;
        if (rank == r0)
            out[0] = v[r];
        if (rank == r1)
            out[1] = v[r];
    }
}

}  // namespace

__global__ __launch_bounds__(kPilotThreads) void pilot_kernel(SampleArgs a)
{
    __shared__ uint32_t buf[2][kPilot];
    __shared__ uint32_t sel[2];
    const int tid = threadIdx.x;
    Status* st = a.st;
    if (tid == 0) {
        st->nB = 0;
        st->solve_state = kSolveNotRun;
        st->emit_done = 0;
        st->nonfinite = 0;
        st->cand_n = 0;
        st->below_n = 0;
        st->ticket_select = 0;
    }
    const int P = a.m < kPilot ? a.m : kPilot;
    uint32_t v[kPilotPer];
#pragma unroll
    for (int r = 0; r < kPilotPer; ++r) {
        const int i = tid * kPilotPer + r;
        v[r] = i < P ? float_to_key(sample_value(a.s, a.n, a.alpha, a.k0, a.k1, (uint32_t)i)) : 0xFFFFFFFFu;
    }
    block_bitonic_regs<kPilotThreads, kPilotPer>(v, buf[0], buf[1]);
    if (tid == 0) {
        sel[0] = 0u;            // open lower bound
        sel[1] = 0xFFFFFFFFu;   // open upper bound
    }
    __syncthreads();
    pick_ranks<kPilotPer>(v, a.pilot_lo >= 1 ? a.pilot_lo : -1, a.pilot_hi <= P ? a.pilot_hi : -1, sel);
    __syncthreads();
    if (tid == 0) {
        st->pilot_lo = sel[0];
        st->pilot_hi = sel[1];
    }
}

// Sort the cnt candidate keys (R per thread, padded with all-ones keys) and
// pick two ranks.
template <int R>
__device__ void select_from(const uint32_t* __restrict__ cand, int cnt, int64_t r0, int64_t r1, uint32_t* buf0,
                            uint32_t* buf1, uint32_t* out)
{
    uint32_t v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = threadIdx.x * R + r;
        v[r] = i < cnt ? cand[i] : 0xFFFFFFFFu;
    }
    block_bitonic_regs<kSelectThreads, R>(v, buf0, buf1);
    pick_ranks<R>(v, r0, r1, out);
}

// The same for the largest candidate counts (targets near the median): a
// bitonic network over LDS, slower but light on registers, so that the
// common shapes above keep their register budget.
__device__ void select_from_lds(const uint32_t* __restrict__ cand, int cnt, int64_t r0, int64_t r1, uint32_t* keys,
                                uint32_t* out)
{
    const int tid = threadIdx.x;
    for (int i = tid; i < kCandCap; i += kSelectThreads)
        keys[i] = i < cnt ? cand[i] : 0xFFFFFFFFu;
    __syncthreads();
    for (int k = 2; k <= kCandCap; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int p = tid; p < kCandCap / 2; p += kSelectThreads) {
                const int i = 2 * p - (p & (j - 1));  // bit log2(j) of i is 0
                const uint32_t x = keys[i], y = keys[i + j];
                if ((x > y) == ((i & k) == 0)) {
                    keys[i] = y;
                    keys[i + j] = x;
                }
            }
            __syncthreads();
        }
    }
    if (tid == 0) {
        if (r0 >= 1 && r0 <= kCandCap)
            out[0] = keys[r0 - 1];
        if (r1 >= 1 && r1 <= kCandCap)
            out[1] = keys[r1 - 1];
    }
}

// Filter and select in one kernel.  Every work-group regenerates its share
// of the samples, counts those below the lower pilot bound and appends those
// between the bounds to the candidate list.  Then it takes a ticket; the
// last work-group to finish (its writes made visible by the release fence
// before each ticket, read after an acquire fence) selects the two target
// order statistics among the candidates.  No work-group waits for another.
__global__ __launch_bounds__(kSelectThreads) void filter_select_kernel(SampleArgs a, SelectArgs se)
{
    constexpr int kWaves = kSelectThreads / kWave;
    __shared__ uint32_t buf[2][kCandCap];
    __shared__ uint32_t sel[2];
    __shared__ uint32_t wcnt[2][kWaves];
    __shared__ uint32_t base_s;
    __shared__ uint32_t is_last;
    Status* st = a.st;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    // ---- filter ------------------------------------------------------------
    {
        const int32_t j = blockIdx.x * kSelectThreads + tid;
        const bool valid = j < a.m;
        const uint32_t key = valid ? float_to_key(sample_value(a.s, a.n, a.alpha, a.k0, a.k1, (uint32_t)j)) : 0u;
        const uint32_t lo = st->pilot_lo, hi = st->pilot_hi;
        const bool below = valid && key < lo;
        const bool cand = valid && key >= lo && key <= hi;
        const uint64_t bm = __ballot(below);
        const uint64_t cm = __ballot(cand);
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
        if (tid == 0) {
            base_s = tot_c ? atomicAdd(&st->cand_n, tot_c) : 0u;
            if (tot_b)
                atomicAdd(&st->below_n, tot_b);
        }
        __syncthreads();
        if (cand) {
            const uint32_t pos = base_s + woff + rank_in_mask(cm);
            if (pos < (uint32_t)kCandCap)
                a.cand[pos] = key;
        }
    }

    // ---- ticket: the last work-group selects ---------------------------------
    __syncthreads();
    if (tid == 0) {
        fence_agent();  // release this work-group's candidates and counts
        const uint32_t t = atomicAdd(&st->ticket_select, 1u);
        is_last = t == gridDim.x - 1 ? 1u : 0u;
    }
    __syncthreads();
    if (!is_last)
        return;
    fence_agent();  // acquire every work-group's candidates and counts

    const uint64_t cb = st->below_n;
    const uint64_t cc = st->cand_n;
    const uint32_t lo_key = st->pilot_lo, hi_key = st->pilot_hi;
    const int64_t rl = se.r_left, rr = se.r_right;
    const bool overflow = cc > (uint64_t)kCandCap;
    const bool left_inf = rl <= 0;
    const bool right_inf = rr > (int64_t)se.m;
    const bool left_in = !left_inf && (uint64_t)rl > cb && (uint64_t)rl <= cb + cc;
    const bool right_in = !right_inf && (uint64_t)rr > cb && (uint64_t)rr <= cb + cc;
    if (!overflow && (left_in || right_in)) {
        // the sort shape follows the candidate count (uniform branch)
        const int cnt = (int)cc;
        const int64_t r0 = left_in ? rl - (int64_t)cb : -1;
        const int64_t r1 = right_in ? rr - (int64_t)cb : -1;
        if (cnt <= kSelectThreads)
            select_from<1>(se.cand, cnt, r0, r1, buf[0], buf[1], sel);
        else if (cnt <= 2 * kSelectThreads)
            select_from<2>(se.cand, cnt, r0, r1, buf[0], buf[1], sel);
        else if (cnt <= 4 * kSelectThreads)
            select_from<4>(se.cand, cnt, r0, r1, buf[0], buf[1], sel);
        else if (cnt <= 8 * kSelectThreads)
            select_from<8>(se.cand, cnt, r0, r1, buf[0], buf[1], sel);
        else
            select_from_lds(se.cand, cnt, r0, r1, buf[0], sel);
    }
    __syncthreads();
    if (tid == 0) {
        // open pilot bounds stand for -inf / +inf
        const float lo_val = lo_key == 0u ? -INFINITY : key_to_float(lo_key);
        const float hi_val = hi_key == 0xFFFFFFFFu ? INFINITY : key_to_float(hi_key);
        uint32_t info = overflow ? 1u : 0u;
        float aL, aR;
        if (left_inf) {
            aL = -INFINITY;
        } else if ((uint64_t)rl <= cb) {
            aL = -INFINITY;  // target below every candidate: open the bracket
            info |= 2u;
        } else if ((uint64_t)rl > cb + cc) {
            aL = hi_val;  // rank cb+cc < r_left: conservative
            info |= 4u;
        } else if (overflow) {
            aL = lo_val;  // rank cb+1 <= r_left: conservative
        } else {
            aL = key_to_float(sel[0]);
        }
        if (right_inf) {
            aR = INFINITY;
        } else if ((uint64_t)rr > cb + cc) {
            aR = INFINITY;  // target above every candidate: open the bracket
            info |= 4u;
        } else if ((uint64_t)rr <= cb) {
            aR = lo_val;  // rank cb+1 >= r_right: conservative
            info |= 2u;
        } else if (overflow) {
            aR = hi_val;  // rank cb+cc >= r_right: conservative
        } else {
            aR = key_to_float(sel[1]);
        }
        st->aL = aL;
        st->aR = aR;
        st->select_info = info;
        st->cand_count = (uint32_t)(cc > 0xFFFFFFFFull ? 0xFFFFFFFFull : cc);
    }
}

hipError_t launch_localize(const SampleArgs& sa, const SelectArgs& se, hipStream_t stream)
{
    STK_LAUNCH(kKPilot, stream, pilot_kernel, dim3(1), dim3(kPilotThreads), 0, stream, sa);
    const int blocks = (sa.m + kSelectThreads - 1) / kSelectThreads;
    STK_LAUNCH(kKSelect, stream, filter_select_kernel, dim3(blocks), dim3(kSelectThreads), 0, stream, sa, se);
    return hipGetLastError();
}

}  // namespace stk
