// partition_solve.hip -- the threshold b without sorting: partition refinement.
//
// Pages: gist.science summary of Fast LapSum, section 2.2 ("Full-Sort
// Solver": between two consecutive scores the budget equation has a closed
// form root; "Probabilistic Bracketing": the band between the bracket ends
// holds b, the tails enter as sums).  The sort of the band is what this file
// replaces.
//
// Split the scores at a point r: N of them lie above r, and
//   A = sum over s_i >  r of e^{-(s_i - r)/alpha}   (every term <= 1)
//   B = sum over s_i <= r of e^{ (s_i - r)/alpha}   (every term <= 1).
// While no score lies strictly between r and b, the mass of the Laplace CDF
// F at b is, with u = e^{(b - r)/alpha},
//   M_r(b) = N - (A/2) u + (B/2) / u,
// the segment's closed form written around r instead of around the
// segment's ends.  M_r(b) = k is a quadratic in u with one positive root,
// taken in its cancellation-free form.
//
// Why repeating the step converges, and exactly.  M_r has M's value and
// slope at r.  A score s that b has crossed enters M_r with the form of the
// wrong side: 1 - cosh((b - s)/alpha) lower than its true term when b > r,
// cosh((s - b)/alpha) - 1 higher when b < r.  So M_r <= M above r and
// M_r >= M below it, and with M decreasing the root b(r) of M_r lies
// between r and the root of M.  The steps r <- b(r) therefore move
// monotonically towards the root and never past it, and the step whose
// interval [r, b(r)] holds no score is the root itself: the closed form on
// the right segment.  Near the root M_r differs from M by the crossed
// scores' cosh terms only, about (rho/6) ((b - r)/alpha)^3 for rho scores
// per alpha, so from a start within an alpha of b three or four passes end
// it.  A step that leaves the bracket proves the same about the root (the
// bound runs one way), which is the bracket certificate.
//
// Arithmetic: every term is 2^{-|s - r| log2(e)/alpha} from the fp64 series
// of exp2_nonpos (relative error ~1e-16), summed in fp64 (all terms
// positive); N is exact.  A score within kIterTol alpha of b on the wrong
// side moves M by at most (kIterTol)^2 / 2 per score, so the convergence
// test accepts it (this also ends the alternation a root that sits exactly
// on a score can cause under rounding).
//
// gfx950 forms:
//   one work-group -- bands up to kIterOneCap values: the band sits in LDS
//     (64 KiB) and every pass is one sweep of it plus one work-group
//     reduction (four waves: the reductions' shuffles and LDS folds cost per
//     wave, and measured 4 us a pass with sixteen);
//   several work-groups -- larger bands, or every score when the band
//     overflowed its buffer (kIterGroups work-groups; kIterGroupsAll when
//     the host knows before launch that every score is refined, since its
//     fp64 terms want more waves): a chain of step kernels, each folding the
//     previous step's per-group sums (every work-group the same way, so all
//     agree on the next split point bit for bit), testing convergence and
//     summing its share at the new point; the first also folds the pass-1
//     partials (in its work-group 0); a final one-group kernel folds the
//     last sums if needed and publishes.  The step that finds the end
//     publishes at once; kernels after it return at once.  No grid barrier,
//     ticket or fence.  A launch in this chain costs 4-5 us whatever it
//     does (measured), so the host sizes the chain from the passes recent
//     calls took, and a chain that runs out resumes where it stopped.
#include "stk_common.hpp"
#include "stk_layout.hpp"
#include "stk_prof.hpp"
#include "stk_reduce.hpp"

namespace stk {

namespace {

constexpr double kIterTol = 0x1p-30;  // convergence slack, in units of alpha
constexpr int kOneT = kIterOneThreads;
constexpr int kStepT = kIterThreads;

// Partition sums of some scores at a split point r.
struct Split {
    double A, B;
    unsigned long long N;
    float lo, hi;  // largest score <= r, smallest score > r
};

__device__ __forceinline__ Split split_empty()
{
    Split s;
    s.A = 0.0;
    s.B = 0.0;
    s.N = 0ull;
    s.lo = -INFINITY;
    s.hi = INFINITY;
    return s;
}

__device__ __forceinline__ void split_add(Split& a, float v, double r, double c)
{
    const double dv = (double)v - r;
    const bool up = dv > 0.0;
    const double e = exp2_nonpos(-fabs(dv) * c);
    a.A += up ? e : 0.0;
    a.B += up ? 0.0 : e;
    a.N += up ? 1ull : 0ull;
    // compare and select: fminf / fmaxf would quieten both operands first
    // (a NaN score fails both compares; pass-1 has flagged it already)
    a.hi = up && v < a.hi ? v : a.hi;
    a.lo = !up && v > a.lo ? v : a.lo;
}

template <int kThreads>
struct SplitLds {
    double A[kThreads / kWave], B[kThreads / kWave];
    unsigned long long N[kThreads / kWave];
    float lo[kThreads / kWave], hi[kThreads / kWave];
};

// Work-group totals, the same bits in every thread (fixed butterflies, then
// the wave values in wave order).  Two barriers; L is free on return.
template <int kThreads>
__device__ __forceinline__ Split block_split(Split s, SplitLds<kThreads>& L)
{
    constexpr int kW = kThreads / kWave;
    const int wave = threadIdx.x / kWave;
    s.A = wave_sum(s.A);
    s.B = wave_sum(s.B);
    s.N = wave_sum_u64(s.N);
    s.lo = wave_max(s.lo);
    s.hi = wave_min(s.hi);
    if (lane_id() == 0) {
        L.A[wave] = s.A;
        L.B[wave] = s.B;
        L.N[wave] = s.N;
        L.lo[wave] = s.lo;
        L.hi[wave] = s.hi;
    }
    __syncthreads();
    Split t = split_empty();
#pragma unroll 4
    for (int w = 0; w < kW; ++w) {
        t.A += L.A[w];
        t.B += L.B[w];
        t.N += L.N[w];
        t.lo = fmaxf(t.lo, L.lo[w]);
        t.hi = fminf(t.hi, L.hi[w]);
    }
    __syncthreads();
    return t;
}

// The pass-1 tails: scores below a_L (count, sum of e^{(s - a_L)/alpha})
// and at or above a_R (count, sum of e^{-(s - a_R)/alpha}).
struct Tails {
    double SL, SR;
    unsigned long long nL, nR;
};

enum StepState : int { kStepGo = 0 };

struct StepOut {
    double b;
    int state;  // kStepGo, or the SolveState that ends the refinement
};

// One refinement step from the sums s at split point r.  With `band`, the
// sums cover the band only: the tails are added at r (which lies in
// [a_L, a_R)), and a root outside the bracket is a rejection.
__device__ __forceinline__ StepOut refine_step(double r, const Split& s, const Tails& t, bool band, float aL, float aR,
                                               double k, double alpha, double c)
{
    double A = s.A, B = s.B, N = (double)s.N;
    if (band) {
        if (t.nR)
            A += t.SR * exp2_nonpos(-((double)aR - r) * c);
        if (t.nL)
            B += t.SL * exp2_nonpos(-(r - (double)aL) * c);
        N += (double)t.nR;
    }
    const double d = k - N;
    // with d = 0 the discriminant is sqrt(A) sqrt(B): the product A B leaves
    // the normal fp64 range when both sums are small (the split hundreds of
    // alpha from the scores on both sides, b between them); any other d is
    // at least an ulp of k, whose square dwarfs such a product
    const double disc = d != 0.0 ? sqrt(d * d + A * B) : sqrt(A) * sqrt(B);
    const double u = d > 0.0 ? B / (d + disc) : (disc - d) / A;
    StepOut o;
    o.b = r + alpha * log(u);
    o.state = kStepGo;
    if (!(u > 0.0) || !(u < INFINITY) || !isfinite(o.b)) {
        o.state = kSolveIterLimit;  // no usable step (sums out of the fp64 range)
        return o;
    }
    const double tol = kIterTol * alpha;
    const bool in_seg = o.b >= (double)s.lo - tol && o.b <= (double)s.hi + tol;
    // a band step may not leave [a_L, a_R): the tails are split there.  Past
    // an end, the root lies past it too (the bound runs one way), unless the
    // step is the root within the slack
    if (band && o.b < (double)aL) {
        o.state = in_seg && o.b >= (double)aL - tol ? kSolveOk : kSolveRejectLow;
        return o;
    }
    if (band && o.b >= (double)aR) {
        o.state = in_seg && o.b <= (double)aR + tol ? kSolveOk : kSolveRejectHigh;
        return o;
    }
    if (in_seg)
        o.state = kSolveOk;
    return o;
}

// The first split point of the one-group form: the middle of the bracket,
// an open end replaced by the band's range (r must lie in [a_L, a_R)).
__device__ __forceinline__ bool start_point(float aL, float aR, uint64_t nB, const Pass1Partial& t, double* r)
{
    const double L = aL > -INFINITY ? (double)aL : (nB ? (double)t.bmin : -INFINITY);
    const double R = aR < INFINITY ? (double)aR : (nB ? (double)t.bmax : INFINITY);
    if (L > -INFINITY && R < INFINITY)
        *r = 0.5 * (L + R);  // < a_R: the midpoint of two distinct floats, or of band values below a_R
    else if (L > -INFINITY)
        *r = L;
    else if (R < INFINITY)
        *r = aR < INFINITY ? nextafter((double)aR, -INFINITY) : R;
    else
        return false;
    return true;
}

__device__ __forceinline__ void finish_refine(const IterArgs& a, const StepOut& o, int passes)
{
    Status* st = a.st;
    if (o.state == kSolveOk) {
        *a.out_b = o.b;
        st->b = o.b;
    }
    st->solve_state = (uint32_t)o.state;
    st->iter_steps = (uint32_t)passes;
}

}  // namespace

// ---------------------------------------------------------------------------
// One work-group: fold pass-1, keep the band in registers, refine.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kOneT) void iter_one_kernel(IterArgs a)
{
    __shared__ SplitLds<kOneT> L;
    __shared__ float vb[kIterOneCap];
    Status* st = a.st;
    const int tid = threadIdx.x;
    const uint64_t nB = st->nB;
    const float aL = st->aL, aR = st->aR;
    const int cnt = nB <= (uint64_t)kIterOneCap && nB <= (uint64_t)a.cap ? (int)nB : 0;
    for (int q0 = 0; q0 * kOneT < cnt; q0 += 16) {
        float v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int i = (q0 + q) * kOneT + tid;
            v[q] = i < cnt ? a.band[i] : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q)
            vb[(q0 + q) * kOneT + tid] = v[q];
    }
    // (reduce_pass1's barriers order these LDS stores before the passes)
    const Pass1Partial t = reduce_pass1(a.p1, a.p1_blocks, st);
    if (tid == 0) {
        st->massL = NAN;
        st->massR = NAN;
        st->iter_mode = 0u;
    }
    uint32_t state = kSolveIterLimit;
    double r = 0.0;
    if (t.nonfinite)
        state = kSolveNonfinite;
    else if (nB > (uint64_t)a.cap)
        state = kSolveOverflow;
    else if (nB > (uint64_t)kIterOneCap)
        state = kSolveIterBig;
    else if (start_point(aL, aR, nB, t, &r)) {
        const Tails tl{t.SL, t.SR, t.nL, t.nR};
        const double c = a.log2e_over_alpha;
        for (int pass = 1; pass <= kIterOneMax; ++pass) {
            Split s = split_empty();
#pragma unroll 4
            for (int i = tid; i < cnt; i += kOneT)
                split_add(s, vb[i], r, c);
            s = block_split<kOneT>(s, L);
            const StepOut o = refine_step(r, s, tl, true, aL, aR, a.k, a.alpha, c);
            if (o.state != kStepGo) {
                if (tid == 0)
                    finish_refine(a, o, pass);
                state = (uint32_t)o.state;
                break;
            }
            r = o.b;
        }
    }
    if (tid == 0 && state != kSolveOk && state != kSolveRejectLow && state != kSolveRejectHigh)
        st->solve_state = state;
    __syncthreads();
    publish_status(st, a.mirror, a.seq);
}

// ---------------------------------------------------------------------------
// Several work-groups.
// ---------------------------------------------------------------------------
namespace {

// The first split point of the step kernels, from the bracket alone (every
// work-group of step 0 takes it before any fold): its middle; with one end
// open, the other end (just below a_R); with both open, 0 (any start
// converges, a far one in more passes).
__device__ __forceinline__ double step_start(float aL, float aR)
{
    if (aL > -INFINITY && aR < INFINITY)
        return 0.5 * ((double)aL + (double)aR);
    if (aL > -INFINITY)
        return (double)aL;
    if (aR < INFINITY)
        return nextafter((double)aR, -INFINITY);
    return 0.0;
}

__device__ __forceinline__ Split load_split(const SplitPartial* p)
{
    const SplitPartial q = *p;
    Split s;
    s.A = q.A;
    s.B = q.B;
    s.N = q.N;
    s.lo = q.lo;
    s.hi = q.hi;
    return s;
}

// This thread's share of a step's partials (work-groups tid, tid +
// kStepT, ...), in a fixed order.
__device__ __forceinline__ Split load_splits(const SplitPartial* part, int groups)
{
    Split s = split_empty();
    for (int g = threadIdx.x; g < groups; g += kStepT) {
        const Split q = load_split(&part[g]);
        s.A += q.A;
        s.B += q.B;
        s.N += q.N;
        s.lo = fmaxf(s.lo, q.lo);
        s.hi = fminf(s.hi, q.hi);
    }
    return s;
}

}  // namespace

// Step `step` of a chain of `steps`.  Step 0 sums every work-group's share
// at the first split point (the bracket's, or where an earlier chain
// stopped when `resume`); its work-group 0 also folds the pass-1 partials
// into the status block and resets the state.  A later step, unless the
// refinement has ended, folds the sums of step - 1 (taken at x[(step-1)&1])
// into the next split point, ends if that is the root or leaves the
// bracket (work-group 0 records the outcome and publishes the status at
// once, so the host need not wait for the remaining steps), else records
// it in x[step & 1] (work-group 0) and sums this work-group's share there.
__global__ __launch_bounds__(kStepT) void iter_step_kernel(IterArgs a, int step, int resume)
{
    constexpr int kPre = 8;  // band values per thread loaded before the fold
    __shared__ SplitLds<kStepT> L;
    Status* st = a.st;
    IterState* is = a.is;
    const int tid = threadIdx.x;
    const int prev = (step - 1) & 1, cur = step & 1;
    // the loads that do not depend on the fold go first: the state and the
    // previous step's sums, then this work-group's first band values
    const uint32_t done = step > 0 ? is->done : 0u;
    const uint64_t nB = st->nB;
    const float aL = st->aL, aR = st->aR;
    Split s = split_empty();
    if (step > 0)
        s = load_splits(&a.part[prev * kIterGroupsAll], a.groups);
    if (done)
        return;
    const bool band = nB <= (uint64_t)a.cap;
    const int64_t nBand = band ? (int64_t)nB : 0;
    const int64_t stride = (int64_t)gridDim.x * kStepT;
    const int64_t i0 = (int64_t)blockIdx.x * kStepT + tid;
    float pre[kPre];
#pragma unroll
    for (int q = 0; q < kPre; ++q) {
        const int64_t i = i0 + q * stride;
        pre[q] = i < nBand ? a.band[i] : 0.0f;
    }
    const double c = a.log2e_over_alpha;
    double r;
    if (step == 0) {
        r = resume ? is->resume_x : step_start(aL, aR);
        if (blockIdx.x == 0) {
            const Pass1Partial t = reduce_pass1(a.p1, a.p1_blocks, st);
            if (tid == 0) {
                st->massL = NAN;
                st->massR = NAN;
                st->iter_mode = band ? 0u : 1u;
                st->solve_state = t.nonfinite ? kSolveNonfinite : kSolveNotRun;
                is->done = t.nonfinite ? 1u : 0u;
                is->x[cur] = r;
            }
        }
    } else {
        const double rp = is->x[prev];
        const Tails tl{st->SL, st->SR, st->nL, st->nR};
        s = block_split<kStepT>(s, L);
        const StepOut o = refine_step(rp, s, tl, band, aL, aR, a.k, a.alpha, c);
        if (o.state != kStepGo) {
            if (blockIdx.x == 0) {
                if (tid == 0) {
                    finish_refine(a, o, a.passes_before + step);
                    is->done = 1u;
                }
                __syncthreads();
                publish_status(st, a.mirror, a.seq);
            }
            return;
        }
        r = o.b;
        if (blockIdx.x == 0 && tid == 0)
            is->x[cur] = r;
    }
    s = split_empty();
    if (band) {
#pragma unroll
        for (int q = 0; q < kPre; ++q)
            if (i0 + q * stride < nBand)
                split_add(s, pre[q], r, c);
        for (int64_t i = i0 + kPre * stride; i < nBand; i += stride)
            split_add(s, a.band[i], r, c);
    } else {
        // whole float4 when the vector is 16-byte aligned, single floats after
        const bool vec = (reinterpret_cast<uintptr_t>(a.s) & 15u) == 0;
        const int64_t n4 = vec ? a.n / 4 : 0;
        const float4* s4 = reinterpret_cast<const float4*>(a.s);
        // four loads in flight per lane (one work-group per CU leaves little
        // else to hide their latency), then their sixteen terms
        constexpr int kQ = 4;
        int64_t i = i0;
        for (; i + (kQ - 1) * stride < n4; i += kQ * stride) {
            float4 q[kQ];
#pragma unroll
            for (int u = 0; u < kQ; ++u)
                q[u] = s4[i + u * stride];
#pragma unroll
            for (int u = 0; u < kQ; ++u) {
                split_add(s, q[u].x, r, c);
                split_add(s, q[u].y, r, c);
                split_add(s, q[u].z, r, c);
                split_add(s, q[u].w, r, c);
            }
        }
        for (; i < n4; i += stride) {
            const float4 q = s4[i];
            split_add(s, q.x, r, c);
            split_add(s, q.y, r, c);
            split_add(s, q.z, r, c);
            split_add(s, q.w, r, c);
        }
        for (int64_t i = 4 * n4 + i0; i < a.n; i += stride)
            split_add(s, a.s[i], r, c);
    }
    s = block_split<kStepT>(s, L);
    if (tid == 0) {
        SplitPartial q;
        q.A = s.A;
        q.B = s.B;
        q.N = s.N;
        q.lo = s.lo;
        q.hi = s.hi;
        a.part[cur * kIterGroupsAll + blockIdx.x] = q;
    }
}

// After `steps` steps: unless the refinement has ended, fold the last sums
// and record the outcome -- the root, a rejection, no usable step
// (kSolveIterLimit), or the next split point with kSolveIterMore when the
// steps ran out first (a further chain resumes there) -- and publish the
// status (again, if a step has published it: the same words).
__global__ __launch_bounds__(kStepT) void iter_final_kernel(IterArgs a, int steps)
{
    __shared__ SplitLds<kStepT> L;
    Status* st = a.st;
    IterState* is = a.is;
    const int tid = threadIdx.x;
    if (!is->done) {
        const int last = (steps - 1) & 1;
        const uint64_t nB = st->nB;
        const bool band = nB <= (uint64_t)a.cap;
        Split s = load_splits(&a.part[last * kIterGroupsAll], a.groups);
        const Tails tl{st->SL, st->SR, st->nL, st->nR};
        s = block_split<kStepT>(s, L);
        StepOut o = refine_step(is->x[last], s, tl, band, st->aL, st->aR, a.k, a.alpha, a.log2e_over_alpha);
        if (tid == 0) {
            if (o.state == kStepGo) {
                is->resume_x = o.b;
                o.state = kSolveIterMore;
            }
            finish_refine(a, o, a.passes_before + steps);
        }
    }
    __syncthreads();
    publish_status(st, a.mirror, a.seq);
}

hipError_t launch_partition_solve(const IterArgs& a, bool one_group, int steps, bool resume, hipStream_t stream)
{
    if (one_group) {
        STK_LAUNCH(kKIterate, stream, iter_one_kernel, dim3(1), dim3(kOneT), 0, stream, a);
        return hipGetLastError();
    }
    for (int j = 0; j < steps; ++j)
        STK_LAUNCH(kKIterate, stream, iter_step_kernel, dim3(a.groups), dim3(kStepT), 0, stream, a, j, resume ? 1 : 0);
    STK_LAUNCH(kKIterate, stream, iter_final_kernel, dim3(1), dim3(kStepT), 0, stream, a, steps);
    return hipGetLastError();
}

}  // namespace stk
