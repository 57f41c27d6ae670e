// pass1.hip -- the streaming and filtering pass of the bracketed solver.
//
// gist.science summary of Fast LapSum, section 2.2, "Probabilistic
// Bracketing" step 2: the whole score vector is streamed once; scores
// outside [a_L, a_R) are folded into tail sums, and only the middle band is
// kept.  Here, for every score s:
//   s <  a_L : nL += 1, SL += e^{(s - a_L)/alpha}      (exponent <= 0)
//   s >= a_R : nR += 1, SR += e^{-(s - a_R)/alpha}     (exponent <= 0)
//   else     : s is appended to the band.
// Both tails then enter the solve as two virtual nodes: for any b in
// [a_L, a_R] the left tail contributes SL e^{(a_L - b)/alpha} / 2 to M(b) and
// the right tail nR - SR e^{-(a_R - b)/alpha} / 2.
//
// Design for gfx950: one work-group per contiguous chunk, 16-byte loads,
// per-lane fp64 accumulators, band elements appended with one ballot and one
// LDS atomic per wave into a 16 KiB LDS stage that is flushed with a single
// global atomic per work-group, then a deterministic two-level reduction
// (wave butterflies, a fixed-order pass over the per-group partials by the
// last work-group to finish).
#include "stk_common.hpp"
#include "stk_layout.hpp"
#include "stk_prof.hpp"
#include "stk_reduce.hpp"

namespace stk {

namespace {

struct Acc {
    double SL, SR;
    uint32_t nL, nR;
    float bmin, bmax, smin, smax;
    uint32_t nonfinite;
};

struct Stage {
    float* buf;        // LDS, kStageCap
    uint32_t* count;   // LDS reservation counter
};

// Classify one score, accumulate tails, and append band members.  Called by
// every lane of the wave (valid=false lanes contribute nothing), so the
// ballot sees the whole wave.
__device__ __forceinline__ void visit(float v, bool valid, float aL, float aR, double daL, double daR,
                                      double c, Acc& acc, const Stage& stg, float* __restrict__ band,
                                      int64_t cap, uint64_t* nB_global)
{
    const bool left = valid && (v < aL);
    const bool right = valid && (v >= aR);
    const bool in_band = valid && !left && !right;
    if (valid) {
        acc.nonfinite |= is_nonfinite(v) ? 1u : 0u;
        acc.smin = fminf(acc.smin, v);
        acc.smax = fmaxf(acc.smax, v);
    }
    const double x = left ? ((double)v - daL) : ((double)daR - (double)v);
    const double y = (left || right) ? x * c : -2000.0;
    const double e = exp2_nonpos(y);
    acc.SL += left ? e : 0.0;
    acc.SR += right ? e : 0.0;
    acc.nL += left ? 1u : 0u;
    acc.nR += right ? 1u : 0u;
    if (in_band) {
        acc.bmin = fminf(acc.bmin, v);
        acc.bmax = fmaxf(acc.bmax, v);
    }

    const uint64_t mask = __ballot(in_band);
    if (mask == 0)
        return;
    const uint32_t total = (uint32_t)__popcll(mask);
    const uint64_t active = __ballot(1);
    const int leader = __ffsll((long long)active) - 1;
    const int lane = lane_id();
    uint32_t base = 0;
    if (lane == leader)
        base = atomicAdd(stg.count, total);
    base = __shfl(base, leader, kWave);
    const uint32_t pos = base + rank_in_mask(mask);
    // reservations past the LDS stage go straight to the global band
    const uint32_t first_over = base > (uint32_t)kStageCap ? base : (uint32_t)kStageCap;
    const uint32_t end = base + total;
    const uint32_t n_over = end > first_over ? end - first_over : 0u;
    unsigned long long gbase = 0;
    if (n_over) {
        if (lane == leader)
            gbase = atomicAdd((unsigned long long*)nB_global, (unsigned long long)n_over);
        gbase = __shfl(gbase, leader, kWave);
    }
    if (in_band) {
        if (pos < (uint32_t)kStageCap) {
            stg.buf[pos] = v;
        } else {
            const uint64_t g = (uint64_t)gbase + (pos - first_over);
            if (g < (uint64_t)cap)
                band[g] = v;
        }
    }
}

}  // namespace

template <bool kVec>
__global__ __launch_bounds__(kStreamThreads) void pass1_kernel(Pass1Args a)
{
    __shared__ float stage_buf[kStageCap];
    __shared__ uint32_t stage_count;
    __shared__ unsigned long long stage_base;
    __shared__ double red_d[2][kStreamThreads / kWave];
    __shared__ uint32_t red_u[3][kStreamThreads / kWave];
    __shared__ float red_f[4][kStreamThreads / kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    Status* st = a.st;

    if (tid == 0)
        stage_count = 0;
    __syncthreads();

    const float aL = st->aL;
    const float aR = st->aR;
    const double daL = aL, daR = aR;
    const double c = a.log2e_over_alpha;
    Stage stg{stage_buf, &stage_count};
    uint64_t* nB = &st->nB;

    Acc acc{0.0, 0.0, 0u, 0u, INFINITY, -INFINITY, INFINITY, -INFINITY, 0u};

    const int64_t n4 = a.n >> 2;
    const int64_t q0 = (n4 * blockIdx.x) / a.blocks;
    const int64_t q1 = (n4 * (blockIdx.x + 1)) / a.blocks;
    const float4* s4 = reinterpret_cast<const float4*>(a.s);

    // main loop: four 16-byte loads in flight per lane; the trip count is
    // the same for every lane, so the ballots below see whole waves
    int64_t qb = q0;
    for (; qb + 4 * kStreamThreads <= q1; qb += 4 * kStreamThreads) {
        const int64_t q = qb + tid;
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (kVec) {
                v[u] = s4[q + u * kStreamThreads];
            } else {
                const float* p = a.s + 4 * (q + u * kStreamThreads);
                v[u] = make_float4(p[0], p[1], p[2], p[3]);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            visit(v[u].x, true, aL, aR, daL, daR, c, acc, stg, a.band, a.cap, nB);
            visit(v[u].y, true, aL, aR, daL, daR, c, acc, stg, a.band, a.cap, nB);
            visit(v[u].z, true, aL, aR, daL, daR, c, acc, stg, a.band, a.cap, nB);
            visit(v[u].w, true, aL, aR, daL, daR, c, acc, stg, a.band, a.cap, nB);
        }
    }
    // remainder of the chunk; out-of-range lanes visit with valid=false
    for (; qb < q1; qb += kStreamThreads) {
        const int64_t qq = qb + tid;
        const bool valid = qq < q1;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (valid) {
            if (kVec) {
                v = s4[qq];
            } else {
                const float* p = a.s + 4 * qq;
                v = make_float4(p[0], p[1], p[2], p[3]);
            }
        }
        visit(v.x, valid, aL, aR, daL, daR, c, acc, stg, a.band, a.cap, nB);
        visit(v.y, valid, aL, aR, daL, daR, c, acc, stg, a.band, a.cap, nB);
        visit(v.z, valid, aL, aR, daL, daR, c, acc, stg, a.band, a.cap, nB);
        visit(v.w, valid, aL, aR, daL, daR, c, acc, stg, a.band, a.cap, nB);
    }
    // the last 0..3 scores when n is not a multiple of 4
    if (blockIdx.x == a.blocks - 1 && wave == 0) {
        const int64_t i = 4 * n4 + lane;
        const bool valid = lane < 4 && i < a.n;
        const float v = valid ? a.s[i] : 0.f;
        visit(v, valid, aL, aR, daL, daR, c, acc, stg, a.band, a.cap, nB);
    }

    // flush the LDS stage with one global reservation
    __syncthreads();
    const uint32_t staged = stage_count < (uint32_t)kStageCap ? stage_count : (uint32_t)kStageCap;
    if (tid == 0)
        stage_base = staged ? atomicAdd((unsigned long long*)nB, (unsigned long long)staged) : 0ull;
    __syncthreads();
    for (uint32_t i = tid; i < staged; i += kStreamThreads) {
        const uint64_t g = (uint64_t)stage_base + i;
        if (g < (uint64_t)a.cap)
            a.band[g] = stage_buf[i];
    }

    // work-group reduction into this group's partial; the consumer (segment
    // solve or finalize kernel) folds the partials in fixed order.  No
    // ticket: an agent-scope fence per work-group would write back the whole
    // L2 each time.
    double SL = wave_sum(acc.SL);
    double SR = wave_sum(acc.SR);
    uint32_t nL = wave_sum_u32(acc.nL);
    uint32_t nR = wave_sum_u32(acc.nR);
    uint32_t nf = acc.nonfinite;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        nf |= __shfl_xor(nf, off, kWave);
    const float bmin = wave_min(acc.bmin), bmax = wave_max(acc.bmax);
    const float smin = wave_min(acc.smin), smax = wave_max(acc.smax);
    if (lane == 0) {
        red_d[0][wave] = SL;
        red_d[1][wave] = SR;
        red_u[0][wave] = nL;
        red_u[1][wave] = nR;
        red_u[2][wave] = nf;
        red_f[0][wave] = bmin;
        red_f[1][wave] = bmax;
        red_f[2][wave] = smin;
        red_f[3][wave] = smax;
    }
    __syncthreads();
    if (tid == 0) {
        Pass1Partial p;
        p.SL = 0.0;
        p.SR = 0.0;
        p.nL = 0;
        p.nR = 0;
        p.nonfinite = 0;
        p.bmin = INFINITY;
        p.bmax = -INFINITY;
        p.smin = INFINITY;
        p.smax = -INFINITY;
        for (int w = 0; w < kStreamThreads / kWave; ++w) {
            p.SL += red_d[0][w];
            p.SR += red_d[1][w];
            p.nL += red_u[0][w];
            p.nR += red_u[1][w];
            p.nonfinite |= red_u[2][w];
            p.bmin = fminf(p.bmin, red_f[0][w]);
            p.bmax = fmaxf(p.bmax, red_f[1][w]);
            p.smin = fminf(p.smin, red_f[2][w]);
            p.smax = fmaxf(p.smax, red_f[3][w]);
        }
        a.partials[blockIdx.x] = p;
    }
}

__global__ __launch_bounds__(kStreamThreads) void pass1_finalize_kernel(const Pass1Partial* partials, int blocks,
                                                                        Status* st)
{
    reduce_pass1(partials, blocks, st);
}

hipError_t launch_pass1_finalize(const Pass1Partial* partials, int blocks, Status* st, hipStream_t stream)
{
    STK_LAUNCH(kKReset, stream, pass1_finalize_kernel, dim3(1), dim3(kStreamThreads), 0, stream, partials, blocks, st);
    return hipGetLastError();
}

hipError_t launch_pass1(const Pass1Args& a, hipStream_t stream)
{
    const bool vec = (reinterpret_cast<uintptr_t>(a.s) & 15u) == 0;
    if (vec)
        STK_LAUNCH(kKPass1, stream, pass1_kernel<true>, dim3(a.blocks), dim3(kStreamThreads), 0, stream, a);
    else
        STK_LAUNCH(kKPass1, stream, pass1_kernel<false>, dim3(a.blocks), dim3(kStreamThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace stk
