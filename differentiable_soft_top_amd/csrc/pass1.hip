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
// Design for gfx950: one work-group per contiguous chunk, sixteen scores per
// lane per step (four 16-byte loads in flight).  Classification is fp32
// compares only.  A tail score contributes 2^y with y = -|s - a|/alpha*log2e;
// below y = -50 the term is under 2^-50 and is dropped (all dropped terms
// together stay below n * 2^-50 < 2e-6, far under the mass tolerance), so only
// "near" tail scores need the fp64 exponential.  Each lane queues its near
// scores in its own LDS list and the wave then runs the exponential over the
// queues with every lane busy, instead of paying it for every score.  Band
// scores are queued in the same per-lane list (from the other end) and
// appended with one LDS reservation per wave and step into a work-group
// stage, flushed with one global reservation per work-group.  Counts are
// exact; sums are fp64; per-group partials are folded in fixed order by the
// consumer.
#include "stk_common.hpp"
#include "stk_layout.hpp"
#include "stk_prof.hpp"
#include "stk_reduce.hpp"

namespace stk {

namespace {

constexpr int kVals = 16;           // scores per lane per step
constexpr int kLaneSlots = 17;      // per-lane LDS list (stride 17: no bank conflicts)
constexpr double kTailCut = 50.0;   // tail terms below 2^-50 are dropped
constexpr int kP1Stage = 2048;      // band scores staged per work-group

struct Lanes {
    float* stage;                   // LDS [kP1Stage]
    uint32_t* stage_count;          // LDS reservation counter
    float* my;                      // this lane's LDS list [kLaneSlots]
};

struct Ctx1 {
    float aL, aR, tL, tR;
    double daL, daR, c;
    bool open;                      // a bracket end is infinite: track the band range
    float* band;
    int64_t cap;
    unsigned long long* nB;
};

struct Acc1 {
    double SL, SR;
    uint32_t nL, nR;
    float bmin, bmax;
    float nf;                       // stays 0 unless a score is NaN or +-inf
};

// Classify up to 16 scores of this lane (v[i] valid iff bit i of `valid`;
// kAll: all valid), fold near tail scores into the fp64 sums and append band
// scores.  Called by every lane of the wave (the ballots and the reservation
// are per wave).
//
// The per-lane list holds near scores from slot 0 up and band scores from
// slot 16 down; both are stored unconditionally at their next free slot and
// committed by bumping the count, which keeps the classification loop free of
// branches (a speculative store only ever lands on a free slot: after i
// scores nn + nb <= i, so the next near slot nn and the next band slot 16-nb
// never reach a committed entry of the other list).
template <bool kAll>
__device__ __forceinline__ void step16(const float (&v)[kVals], uint32_t valid, const Ctx1& x, Acc1& acc,
                                       const Lanes& L)
{
    uint32_t nn = 0, nb = 0;
#pragma unroll
    for (int i = 0; i < kVals; ++i) {
        const bool ok = kAll || ((valid >> i) & 1u);
        const float s = v[i];
        const bool left = ok && s < x.aL;
        const bool right = ok && s >= x.aR;
        const bool band = ok && !(s < x.aL) && !(s >= x.aR);
        acc.nL += left ? 1u : 0u;
        acc.nR += right ? 1u : 0u;
        const bool near = (left && s >= x.tL) || (right && s < x.tR);
        L.my[nn] = s;
        nn += near ? 1u : 0u;
        L.my[kLaneSlots - 1 - nb] = s;
        nb += band ? 1u : 0u;
        acc.nf = fmaf(s, 0.f, acc.nf);
    }
    // fp64 exponentials of the queued near scores, every lane busy
    for (uint32_t j = 0; __ballot(j < nn) != 0; ++j) {
        if (j < nn) {
            const float s = L.my[j];
            const bool left = s < x.aL;
            const double d = left ? (double)s - x.daL : x.daR - (double)s;
            const double e = exp2_nonpos(d * x.c);
            if (left)
                acc.SL += e;
            else
                acc.SR += e;
        }
    }
    // band append: lane offsets from the bit planes of nb (<= 16)
    uint32_t prefix = 0, total = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b) {
        const uint64_t m = __ballot((nb >> b) & 1u);
        prefix += rank_in_mask(m) << b;
        total += (uint32_t)__popcll(m) << b;
    }
    if (total == 0)
        return;
    const int lane = lane_id();
    uint32_t base = 0;
    if (lane == 0)
        base = atomicAdd(L.stage_count, total);
    base = __shfl(base, 0, kWave);
    // reservations past the LDS stage go straight to the global band
    const uint32_t first_over = base > (uint32_t)kP1Stage ? base : (uint32_t)kP1Stage;
    const uint32_t end = base + total;
    const uint32_t n_over = end > first_over ? end - first_over : 0u;
    unsigned long long gbase = 0;
    if (n_over) {
        if (lane == 0)
            gbase = atomicAdd(x.nB, (unsigned long long)n_over);
        gbase = __shfl(gbase, 0, kWave);
    }
    for (uint32_t k = 0; k < nb; ++k) {
        const uint32_t pos = base + prefix + k;
        const float s = L.my[kLaneSlots - 1 - k];
        if (x.open) {
            acc.bmin = fminf(acc.bmin, s);
            acc.bmax = fmaxf(acc.bmax, s);
        }
        if (pos < (uint32_t)kP1Stage) {
            L.stage[pos] = s;
        } else {
            const uint64_t g = (uint64_t)gbase + (pos - first_over);
            if (g < (uint64_t)x.cap)
                x.band[g] = s;
        }
    }
}

}  // namespace

template <bool kVec>
__global__ __launch_bounds__(kStreamThreads) void pass1_kernel(Pass1Args a)
{
    __shared__ float stage_buf[kP1Stage];
    __shared__ float lists[kStreamThreads * kLaneSlots];
    __shared__ uint32_t stage_count;
    __shared__ unsigned long long stage_base;
    __shared__ double red_d[2][kStreamThreads / kWave];
    __shared__ uint32_t red_u[3][kStreamThreads / kWave];
    __shared__ float red_f[2][kStreamThreads / kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    Status* st = a.st;

    if (tid == 0)
        stage_count = 0;
    __syncthreads();

    Ctx1 x;
    x.aL = st->aL;
    x.aR = st->aR;
    x.daL = x.aL;
    x.daR = x.aR;
    x.c = a.log2e_over_alpha;
    // near thresholds in fp32, rounded outward so no term >= 2^-50 is dropped
    const double cut = kTailCut / x.c;
    x.tL = (float)(x.daL - cut);
    if ((double)x.tL > x.daL - cut)
        x.tL = nextafterf(x.tL, -INFINITY);
    x.tR = (float)(x.daR + cut);
    if ((double)x.tR < x.daR + cut)
        x.tR = nextafterf(x.tR, INFINITY);
    x.open = (x.aL == -INFINITY) || (x.aR == INFINITY);
    x.band = a.band;
    x.cap = a.cap;
    x.nB = reinterpret_cast<unsigned long long*>(&st->nB);
    Lanes L{stage_buf, &stage_count, lists + tid * kLaneSlots};

    Acc1 acc{0.0, 0.0, 0u, 0u, INFINITY, -INFINITY, 0.f};

    const int64_t n4 = a.n >> 2;
    const int64_t q0 = (n4 * blockIdx.x) / a.blocks;
    const int64_t q1 = (n4 * (blockIdx.x + 1)) / a.blocks;
    const float4* s4 = reinterpret_cast<const float4*>(a.s);

    // uniform trip count: every lane runs every step (ballots see whole waves)
    int64_t qb = q0;
    for (; qb + 4 * kStreamThreads <= q1; qb += 4 * kStreamThreads) {
        float v[kVals];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t q = qb + u * kStreamThreads + tid;
            float4 f;
            if (kVec) {
                f = s4[q];
            } else {
                const float* p = a.s + 4 * q;
                f = make_float4(p[0], p[1], p[2], p[3]);
            }
            v[4 * u + 0] = f.x;
            v[4 * u + 1] = f.y;
            v[4 * u + 2] = f.z;
            v[4 * u + 3] = f.w;
        }
        step16<true>(v, 0xFFFFu, x, acc, L);
    }
    if (qb < q1) {
        float v[kVals];
        uint32_t valid = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t q = qb + u * kStreamThreads + tid;
            float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
            if (q < q1) {
                if (kVec) {
                    f = s4[q];
                } else {
                    const float* p = a.s + 4 * q;
                    f = make_float4(p[0], p[1], p[2], p[3]);
                }
                valid |= 0xFu << (4 * u);
            }
            v[4 * u + 0] = f.x;
            v[4 * u + 1] = f.y;
            v[4 * u + 2] = f.z;
            v[4 * u + 3] = f.w;
        }
        step16<false>(v, valid, x, acc, L);
    }
    // the last 0..3 scores when n is not a multiple of 4
    if (blockIdx.x == a.blocks - 1) {
        const int64_t i = 4 * n4 + tid;
        float v[kVals];
#pragma unroll
        for (int k = 0; k < kVals; ++k)
            v[k] = 0.f;
        uint32_t valid = 0;
        if (tid < 4 && i < a.n) {
            v[0] = a.s[i];
            valid = 1u;
        }
        step16<false>(v, valid, x, acc, L);
    }

    // flush the LDS stage with one global reservation
    __syncthreads();
    const uint32_t staged = stage_count < (uint32_t)kP1Stage ? stage_count : (uint32_t)kP1Stage;
    if (tid == 0)
        stage_base = staged ? atomicAdd(x.nB, (unsigned long long)staged) : 0ull;
    __syncthreads();
    for (uint32_t i = tid; i < staged; i += kStreamThreads) {
        const uint64_t g = (uint64_t)stage_base + i;
        if (g < (uint64_t)a.cap)
            a.band[g] = stage_buf[i];
    }

    // work-group reduction into this group's partial; the consumer (segment
    // solve) folds the partials in fixed order.  No ticket: an agent-scope
    // fence per work-group would write back the whole L2 each time.
    const double SL = wave_sum(acc.SL);
    const double SR = wave_sum(acc.SR);
    const uint32_t nL = wave_sum_u32(acc.nL);
    const uint32_t nR = wave_sum_u32(acc.nR);
    uint32_t nf = acc.nf != 0.f || acc.nf != acc.nf ? 1u : 0u;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        nf |= __shfl_xor(nf, off, kWave);
    const float bmin = wave_min(acc.bmin), bmax = wave_max(acc.bmax);
    if (lane == 0) {
        red_d[0][wave] = SL;
        red_d[1][wave] = SR;
        red_u[0][wave] = nL;
        red_u[1][wave] = nR;
        red_u[2][wave] = nf;
        red_f[0][wave] = bmin;
        red_f[1][wave] = bmax;
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
        }
        a.partials[blockIdx.x] = p;
    }
}

// ---------------------------------------------------------------------------
// Score range and finiteness for the full-sort route (the radix sort only
// sorts the key bits that vary between the smallest and largest score).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kStreamThreads) void range_kernel(const float* __restrict__ s, int64_t n,
                                                               Pass1Partial* partials, int blocks)
{
    __shared__ float red[3][kStreamThreads / kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int64_t i0 = (n * blockIdx.x) / blocks;
    const int64_t i1 = (n * (blockIdx.x + 1)) / blocks;
    float mn = INFINITY, mx = -INFINITY, nf = 0.f;
    for (int64_t i = i0 + tid; i < i1; i += kStreamThreads) {
        const float v = s[i];
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
        nf = fmaf(v, 0.f, nf);
    }
    uint32_t bad = (nf != 0.f || nf != nf) ? 1u : 0u;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        bad |= __shfl_xor(bad, off, kWave);
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
        red[0][wave] = mn;
        red[1][wave] = mx;
        red[2][wave] = bad ? 1.f : 0.f;
    }
    __syncthreads();
    if (tid == 0) {
        Pass1Partial p;
        p.SL = 0.0;
        p.SR = 0.0;
        p.nL = 0;
        p.nR = 0;
        p.bmin = INFINITY;
        p.bmax = -INFINITY;
        p.smin = INFINITY;
        p.smax = -INFINITY;
        p.nonfinite = 0;
        for (int w = 0; w < kStreamThreads / kWave; ++w) {
            p.smin = fminf(p.smin, red[0][w]);
            p.smax = fmaxf(p.smax, red[1][w]);
            p.nonfinite |= red[2][w] != 0.f ? 1u : 0u;
        }
        partials[blockIdx.x] = p;
    }
}

hipError_t launch_range(const float* s, int64_t n, Pass1Partial* partials, int blocks, hipStream_t stream)
{
    STK_LAUNCH(kKPass1, stream, range_kernel, dim3(blocks), dim3(kStreamThreads), 0, stream, s, n, partials, blocks);
    return hipGetLastError();
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
