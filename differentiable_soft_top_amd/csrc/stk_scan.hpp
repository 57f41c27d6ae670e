// stk_scan.hpp -- anchored exponential sums and their work-group scans.
//
// gist.science summary of Fast LapSum, section 2.2, "Full-Sort Solver": on
// sorted data, stable prefix and suffix sums of shifted exponentials give
// the mass at every breakpoint, and a closed form gives the root inside the
// gap where the mass crosses k.  These are the pieces the segment solve and
// the batched-row solve share.
#pragma once

#include "stk_common.hpp"

namespace stk {

namespace {

// An anchored exponential sum: value v anchored at point x.  Every anchor
// is an fp32 score (or a bracket end, itself a sample value), so x is fp32.
// An empty prefix is (x = -inf, v = 0) and an empty suffix (x = +inf, v = 0):
// with the exponential clamped to [0, 1] (exp2_nonpos: NaN and -inf give 0,
// +inf gives 1) the combinations below need no emptiness flag.
struct Anch {
    float x;
    double v;
};

__device__ __forceinline__ Anch node(float x, double v)
{
    Anch a;
    a.x = x;
    a.v = v;
    return a;
}

__device__ __forceinline__ Anch empty_pre() { return node(-INFINITY, 0.0); }
__device__ __forceinline__ Anch empty_suf() { return node(INFINITY, 0.0); }

// prefix: earlier e, later l (x_e <= x_l), anchored at the later point
__device__ __forceinline__ Anch fwd(Anch e, Anch l, double c)
{
    return node(fmaxf(e.x, l.x), l.v + exp2_nonpos_lowdepth(((double)e.x - (double)l.x) * c) * e.v);
}

// suffix: left l, right r (x_l <= x_r), anchored at the left point
__device__ __forceinline__ Anch bwd(Anch l, Anch r, double c)
{
    return node(fminf(l.x, r.x), l.v + exp2_nonpos_lowdepth(((double)l.x - (double)r.x) * c) * r.v);
}

__device__ __forceinline__ Anch shfl_anch(Anch a, int src_lane)
{
    return node(__shfl(a.x, src_lane, kWave), __shfl(a.v, src_lane, kWave));
}

// Work-group scan of two anchored sums per thread: `pre` (this thread's
// items folded forward, anchored at its last point) and `suf` (folded
// backward, anchored at its first point), plus a u32 count.  Each wave scans
// with shuffles (the two directions interleaved so their latencies
// overlap); the wave totals meet in LDS behind one barrier; every wave then
// scans the kSW wave totals with log2(kSW) more shuffle steps.
struct WaveTot {
    double pv, sv;
    float px, sx;
    uint32_t cnt;
};

struct Scan2 {
    Anch pre_before, suf_after, pre_all, suf_all;
    uint32_t cnt_before, cnt_all;
};

struct Scan2Part {
    Anch pw_ex, sw_ex;   // within-wave exclusive values
    uint32_t cw_ex;
};

__device__ __forceinline__ Scan2Part scan2_publish(Anch pre, Anch suf, uint32_t cnt, double c, WaveTot* wt)
{
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    Anch p = pre, q = suf;
    uint32_t n = cnt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const Anch op = shfl_anch(p, lane >= off ? lane - off : lane);
        const Anch oq = shfl_anch(q, lane + off < kWave ? lane + off : lane);
        const uint32_t on = __shfl_up(n, off, kWave);
        if (lane >= off) {
            p = fwd(op, p, c);
            n += on;
        }
        if (lane + off < kWave)
            q = bwd(q, oq, c);
    }
    Scan2Part r;
    r.pw_ex = shfl_anch(p, lane > 0 ? lane - 1 : 0);
    r.sw_ex = shfl_anch(q, lane < kWave - 1 ? lane + 1 : kWave - 1);
    r.cw_ex = n - cnt;
    if (lane == 0)
        r.pw_ex = empty_pre();
    if (lane == kWave - 1)
        r.sw_ex = empty_suf();
    if (lane == kWave - 1) {
        wt[wave].px = p.x;
        wt[wave].pv = p.v;
        wt[wave].cnt = n;
    }
    if (lane == 0) {
        wt[wave].sx = q.x;
        wt[wave].sv = q.v;
    }
    return r;
}

// after the barrier that follows scan2_publish; kSW: the work-group's waves
template <int kSW>
__device__ __forceinline__ Scan2 scan2_finish(const WaveTot* wt, const Scan2Part& part, double c)
{
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    Anch p = empty_pre(), q = empty_suf();
    uint32_t n = 0;
    if (lane < kSW) {
        p = node(wt[lane].px, wt[lane].pv);
        q = node(wt[lane].sx, wt[lane].sv);
        n = wt[lane].cnt;
    }
#pragma unroll
    for (int off = 1; off < kSW; off <<= 1) {
        const Anch op = shfl_anch(p, lane >= off ? lane - off : lane);
        const Anch oq = shfl_anch(q, lane + off < kSW ? lane + off : lane);
        const uint32_t on = __shfl_up(n, off, kWave);
        if (lane >= off && lane < kSW) {
            p = fwd(op, p, c);
            n += on;
        }
        if (lane + off < kSW)
            q = bwd(q, oq, c);
    }
    Anch pb = shfl_anch(p, wave > 0 ? wave - 1 : 0);
    uint32_t nb = __shfl(n, wave > 0 ? wave - 1 : 0, kWave);
    if (wave == 0) {
        pb = empty_pre();
        nb = 0;
    }
    Anch qa = shfl_anch(q, wave + 1 < kSW ? wave + 1 : 0);
    if (wave == kSW - 1)
        qa = empty_suf();
    Scan2 r;
    r.pre_before = fwd(pb, part.pw_ex, c);
    r.pre_all = shfl_anch(p, kSW - 1);
    r.suf_after = bwd(part.sw_ex, qa, c);
    r.suf_all = shfl_anch(q, 0);
    r.cnt_before = nb + part.cw_ex;
    r.cnt_all = __shfl(n, kSW - 1, kWave);
    return r;
}

// Mass at a point x with prefix P (anchored at x), count after C, and the
// suffix S of everything after (anchored at its first point; may be empty).
__device__ __forceinline__ double mass_at(float x, double Pv, double C, Anch S, double c)
{
    return 0.5 * Pv + C - 0.5 * S.v * exp2_nonpos(((double)x - (double)S.x) * c);
}

// Root of A v/2 + C - B w/2 = k on [xlo, xhi] (an empty end has v = 0).
__device__ inline double gap_root(Anch lo, Anch hi, double C, double k, double alpha, double c)
{
    const double cc = C - k;
    const double xlo = lo.x, xhi = hi.x;
    if (cc == 0.0 && lo.v > 0.0 && hi.v > 0.0)
        return 0.5 * (xlo + xhi) + 0.5 * alpha * log(lo.v / hi.v);
    const double g = (lo.v > 0.0 && hi.v > 0.0) ? exp2_nonpos((xlo - xhi) * c) : 0.0;
    const double r = sqrt(cc * cc + lo.v * hi.v * g);
    if (cc > 0.0)
        return xhi + alpha * log((cc + r) / hi.v);
    return xlo - alpha * log((-cc + r) / lo.v);
}

}  // namespace

}  // namespace stk
