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

// One thread per sample.  Counter (j, 0, 0, 0), key (seed lo, seed hi).
// Word 0/1 give a 64-bit uniform u64; the index is the high half of
// u64 * n (unbiased to 2^-64 n, where a 32-bit product would skew indices by
// up to n/2^32).  Word 2 gives u in (0,1) and E = F^{-1}(u).
__global__ __launch_bounds__(256) void sample_kernel(const float* __restrict__ s, int64_t n, float alpha,
                                                     uint32_t k0, uint32_t k1, int32_t m,
                                                     float* __restrict__ out)
{
    const int32_t j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= m)
        return;
    const Philox4 r = philox4x32_10((uint32_t)j, 0u, 0u, 0u, k0, k1);
    const uint64_t u64 = ((uint64_t)r.v[1] << 32) | (uint64_t)r.v[0];
    const uint64_t idx = __umul64hi(u64, (uint64_t)n);  // < n
    const double u = ((double)r.v[2] + 0.5) * (1.0 / 4294967296.0);
    const double e = (u < 0.5) ? log(2.0 * u) : -log(2.0 * (1.0 - u));
    out[j] = (float)((double)s[idx] + (double)alpha * e);
}

hipError_t launch_sample(const float* s, int64_t n, float alpha, uint64_t seed, int32_t m,
                         float* out_samples, Status* st, hipStream_t stream)
{
    (void)st;
    const int blocks = (m + 255) / 256;
    STK_LAUNCH(kKSample, stream, sample_kernel, dim3(blocks), dim3(256), 0, stream, s, n, alpha,
                       (uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32), m, out_samples);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Exact selection of up to two order statistics (1-based ranks r[0], r[1]) of
// cnt u32 keys held in LDS, by the whole work-group: most-significant-digit
// radix select, four 8-bit digits, both targets refined together.  A rank
// outside [1, cnt] is skipped (its output is left untouched).
// ---------------------------------------------------------------------------
__device__ void lds_select2(const uint32_t* keys, int cnt, int64_t r0, int64_t r1, uint32_t* out0, uint32_t* out1)
{
    __shared__ uint32_t hist[2][256];
    __shared__ uint32_t prefix[2];
    __shared__ int64_t rank[2];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    if (tid == 0) {
        prefix[0] = 0;
        prefix[1] = 0;
        rank[0] = r0;
        rank[1] = r1;
    }
    const bool act0 = r0 >= 1 && r0 <= cnt;
    const bool act1 = r1 >= 1 && r1 <= cnt;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        const uint32_t hmask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
        for (int i = tid; i < 512; i += blockDim.x)
            (&hist[0][0])[i] = 0;
        __syncthreads();
        const uint32_t p0 = prefix[0], p1 = prefix[1];
        for (int i = tid; i < cnt; i += blockDim.x) {
            const uint32_t k = keys[i];
            const uint32_t d = (k >> shift) & 0xFFu;
            if (act0 && ((k ^ p0) & hmask) == 0)
                atomicAdd(&hist[0][d], 1u);
            if (act1 && ((k ^ p1) & hmask) == 0)
                atomicAdd(&hist[1][d], 1u);
        }
        __syncthreads();
        // wave t (t = 0, 1) finds the digit holding rank[t]
        if (wave < 2 && (wave == 0 ? act0 : act1)) {
            const int t = wave;
            const uint32_t c0 = hist[t][4 * lane], c1 = hist[t][4 * lane + 1];
            const uint32_t c2 = hist[t][4 * lane + 2], c3 = hist[t][4 * lane + 3];
            const uint32_t mine = c0 + c1 + c2 + c3;
            uint32_t incl = mine;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const uint32_t o = __shfl_up(incl, off, kWave);
                if (lane >= off)
                    incl += o;
            }
            const uint32_t excl = incl - mine;
            const int64_t r = rank[t];
            if ((int64_t)excl < r && r <= (int64_t)incl) {
                int64_t rr = r - excl;
                int d = 4 * lane;
                if (rr > c0) {
                    rr -= c0;
                    ++d;
                    if (rr > c1) {
                        rr -= c1;
                        ++d;
                        if (rr > c2) {
                            rr -= c2;
                            ++d;
                        }
                    }
                }
                rank[t] = rr;
                prefix[t] |= (uint32_t)d << shift;
            }
        }
        __syncthreads();
    }
    if (tid == 0) {
        if (act0)
            *out0 = prefix[0];
        if (act1)
            *out1 = prefix[1];
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Select the r_left-th and r_right-th smallest of the m samples with one
// work-group: two pilot order statistics (from the first kPilot samples) that
// enclose the targets with a wide margin; a count of the samples below the
// lower one; the samples between them gathered into LDS; the targets
// selected among those.  If the gather overflows or a target falls outside
// the candidates, a pilot value with a more conservative rank is used instead
// (the bracket only widens, so the certificate still decides).
//
// Also clears the per-round counters of the status block: this kernel runs
// first in every bracketed round.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSelectThreads) void select_kernel(SelectArgs a)
{
    __shared__ uint32_t pilot[kPilot];
    __shared__ uint32_t cand[kCandCap];
    __shared__ uint32_t cand_n;
    __shared__ uint32_t wave_below[kSelectThreads / kWave];
    __shared__ uint32_t sel[4];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    Status* st = a.st;

    if (tid == 0) {
        cand_n = 0;
        sel[0] = 0u;            // pilot lower bound: open
        sel[1] = 0xFFFFFFFFu;   // pilot upper bound: open
        st->nB = 0;
        st->solve_state = kSolveNotRun;
        st->emit_done = 0;
        st->nonfinite = 0;
    }

    // 1. pilot bounds: two order statistics of the first P samples
    const int P = a.m < kPilot ? a.m : kPilot;
    for (int i = tid; i < P; i += blockDim.x)
        pilot[i] = float_to_key(a.samples[i]);
    __syncthreads();
    lds_select2(pilot, P, a.pilot_lo, a.pilot_hi, &sel[0], &sel[1]);
    const uint32_t lo_key = sel[0];
    const uint32_t hi_key = sel[1];

    // 2. count below / gather candidates (eight loads in flight per thread)
    constexpr int kBatch = 8;
    uint32_t below = 0;
    for (int base = 0; base < a.m; base += kBatch * kSelectThreads) {
        uint32_t key[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int i = base + j * kSelectThreads + tid;
            key[j] = i < a.m ? float_to_key(a.samples[i]) : 0u;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int i = base + j * kSelectThreads + tid;
            const bool valid = i < a.m;
            const bool is_below = valid && key[j] < lo_key;
            const bool is_cand = valid && key[j] >= lo_key && key[j] <= hi_key;
            below += is_below ? 1u : 0u;
            const uint64_t mask = __ballot(is_cand);
            if (mask) {
                const uint32_t cnt = (uint32_t)__popcll(mask);
                uint32_t pos0 = 0;
                if (lane == 0)
                    pos0 = atomicAdd(&cand_n, cnt);
                pos0 = __shfl(pos0, 0, kWave);
                if (is_cand) {
                    const uint32_t pos = pos0 + rank_in_mask(mask);
                    if (pos < (uint32_t)kCandCap)
                        cand[pos] = key[j];
                }
            }
        }
    }
    below = wave_sum_u32(below);
    if (lane == 0)
        wave_below[wave] = below;
    __syncthreads();
    uint64_t cb = 0;
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w)
        cb += wave_below[w];
    const uint64_t cc = cand_n;

    // 3. the targets among the candidates
    const int64_t rl = a.r_left, rr = a.r_right;
    const bool overflow = cc > (uint64_t)kCandCap;
    const bool left_inf = rl <= 0;
    const bool right_inf = rr > (int64_t)a.m;
    const bool left_in = !left_inf && (uint64_t)rl > cb && (uint64_t)rl <= cb + cc;
    const bool right_in = !right_inf && (uint64_t)rr > cb && (uint64_t)rr <= cb + cc;
    if (!overflow && (left_in || right_in))
        lds_select2(cand, (int)cc, left_in ? rl - (int64_t)cb : 0, right_in ? rr - (int64_t)cb : 0, &sel[2],
                    &sel[3]);

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
            aL = key_to_float(sel[2]);
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
            aR = key_to_float(sel[3]);
        }
        st->aL = aL;
        st->aR = aR;
        st->select_info = info;
        st->cand_count = (uint32_t)(cc > 0xFFFFFFFFull ? 0xFFFFFFFFull : cc);
    }
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream)
{
    STK_LAUNCH(kKSelect, stream, select_kernel, dim3(1), dim3(kSelectThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace stk
