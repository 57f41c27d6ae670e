// curve.hip -- the threshold curve of a score vector.
//
// The gist.science summary of Fast LapSum (section 2.2, "Full-Sort Solver")
// obtains the mass at every breakpoint of the sorted scores from stable
// prefix and suffix sums of shifted exponentials, and reads the root off
// the gap where that mass crosses k.  This file exposes the masses
// themselves: for the sorted scores x_0 <= ... <= x_{n-1},
//   M(x_j) = A_j / 2 + (n - 1 - j) - B_j / 2,
//   A_j = sum_{i<=j} e^{(x_i - x_j)/alpha},  B_j = sum_{i>j} e^{(x_j - x_i)/alpha},
// the k a threshold b = x_j would select (non-increasing in j).  Any k's
// root then lies in the gap where the curve crosses k.
//
// gfx950 design: the full-sort route's radix sort and tile summaries (one
// per 4096 sorted values: count, ends, sums anchored at the ends), then
//   curve_scan_kernel -- one work-group of 1024 threads folds the tile
//     summaries into, for every tile, the anchored sums of all tiles before
//     and after it (per-thread chains over contiguous tiles, one work-group
//     scan of anchored sums);
//   curve_kernel -- one work-group per tile (256 threads x 16 values in
//     blocked order): per-thread chains, a work-group scan, the tile's outer
//     sums, then the mass at each value.
// Anchored sums (every exponent <= 0) hold any span of the scores.
#include "stk_common.hpp"
#include "stk_layout.hpp"
#include "stk_prof.hpp"
#include "stk_scan.hpp"

namespace stk {

namespace {

constexpr int kCurveScanThreads = 1024;
constexpr int kCurveThreads = 256;
constexpr int kCurveR = kTile / kCurveThreads;
static_assert(kCurveR * kCurveThreads == kTile, "one work-group per tile");

// anchored sums of everything before / after a tile (kept in the slots the
// segment solve's group scan uses; the curve runs no solve)
struct TileOuter {
    double pv, sv;
    float px, sx;
};
static_assert(sizeof(TileOuter) <= sizeof(GroupScan), "one tile's outer sums fit a group-scan slot");

__global__ __launch_bounds__(kCurveScanThreads) void curve_scan_kernel(CurveArgs a)
{
    constexpr int kW = kCurveScanThreads / kWave;
    __shared__ WaveTot wt[kW];
    const double c = a.log2e_over_alpha;
    const int tid = threadIdx.x;
    const int per = (a.n_tiles + kCurveScanThreads - 1) / kCurveScanThreads;
    const int t0 = tid * per < a.n_tiles ? tid * per : a.n_tiles;
    const int t1 = t0 + per < a.n_tiles ? t0 + per : a.n_tiles;
    // this thread's tiles: the prefix anchored at the last one's high end,
    // the suffix anchored at the first one's low end
    Anch lp = empty_pre(), ls = empty_suf();
    for (int t = t0; t < t1; ++t)
        lp = fwd(lp, node(a.agg[t].hi, a.agg[t].TA), c);
    for (int t = t1 - 1; t >= t0; --t)
        ls = bwd(node(a.agg[t].lo, a.agg[t].TB), ls, c);
    const Scan2Part part = scan2_publish(lp, ls, 0u, c, wt);
    __syncthreads();
    const Scan2 sc = scan2_finish<kW>(wt, part, c);
    TileOuter* ex = static_cast<TileOuter*>(a.ex);
    Anch P = sc.pre_before;
    for (int t = t0; t < t1; ++t) {
        ex[t].px = P.x;
        ex[t].pv = P.v;
        P = fwd(P, node(a.agg[t].hi, a.agg[t].TA), c);
    }
    Anch S = sc.suf_after;
    for (int t = t1 - 1; t >= t0; --t) {
        ex[t].sx = S.x;
        ex[t].sv = S.v;
        S = bwd(node(a.agg[t].lo, a.agg[t].TB), S, c);
    }
}

__global__ __launch_bounds__(kCurveThreads) void curve_kernel(CurveArgs a)
{
    constexpr int kW = kCurveThreads / kWave;
    constexpr int R = kCurveR;
    __shared__ WaveTot wt[kW];
    const double c = a.log2e_over_alpha;
    const int tid = threadIdx.x;
    const int64_t i0 = (int64_t)blockIdx.x * kTile;
    const int64_t e0 = i0 + (int64_t)tid * R;
    const int m = a.n - e0 <= 0 ? 0 : (a.n - e0 < R ? (int)(a.n - e0) : R);
    float x[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        x[r] = r < m ? a.sorted[e0 + r] : 0.0f;
    // backward chain (suffix from each value, anchored there), forward fold
    double bv[R];
    Anch ls = empty_suf();
#pragma unroll
    for (int r = R - 1; r >= 0; --r) {
        if (r < m)
            ls = bwd(node(x[r], 1.0), ls, c);
        bv[r] = ls.v;
    }
    Anch lp = empty_pre();
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (r < m)
            lp = fwd(lp, node(x[r], 1.0), c);
    const Scan2Part part = scan2_publish(lp, ls, 0u, c, wt);
    __syncthreads();
    const Scan2 sc = scan2_finish<kW>(wt, part, c);
    const TileOuter o = static_cast<const TileOuter*>(a.ex)[blockIdx.x];
    Anch A = fwd(node(o.px, o.pv), sc.pre_before, c);        // everything before this run
    const Anch after = bwd(sc.suf_after, node(o.sx, o.sv), c);  // everything after it
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r < m) {
            A = fwd(A, node(x[r], 1.0), c);
            const Anch Bn = r + 1 < m ? bwd(node(x[r + 1], bv[r + 1]), after, c) : after;
            const int64_t j = e0 + r;
            a.out_sorted[j] = x[r];
            a.out_mass[j] = mass_at(x[r], A.v, (double)(a.n - 1 - j), Bn, c);
        }
    }
}

}  // namespace

hipError_t launch_curve(const CurveArgs& a, hipStream_t stream)
{
    STK_LAUNCH(kKCurveScan, stream, curve_scan_kernel, dim3(1), dim3(kCurveScanThreads), 0, stream, a);
    STK_LAUNCH(kKCurve, stream, curve_kernel, dim3((uint32_t)a.n_tiles), dim3(kCurveThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace stk
