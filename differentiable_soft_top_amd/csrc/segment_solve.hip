// segment_solve.hip -- exact threshold from sorted data ("threshold curve").
//
// gist.science summary of Fast LapSum, section 2.2, "Full-Sort Solver": after
// sorting, one numerically stable prefix/suffix scan of shifted exponential
// sums gives the mass at every breakpoint; an index lookup finds the interval
// where sum p = k balances and a closed-form root inside it gives b.  Step 3
// of the bracketed pipeline applies the same solver to the middle band, with
// the tails entering as two virtual end nodes.
//
// Notation (x sorted ascending, alpha the temperature):
//   A_j = sum_{i<=j} e^{(x_i - x_j)/alpha}   (prefix anchored at x_j, <= j)
//   B_j = sum_{i>=j} e^{-(x_i - x_j)/alpha}  (suffix anchored at x_j)
//   M(x_j) = A_j/2 + C_j - B_{j+1} e^{-(x_{j+1} - x_j)/alpha}/2,
//            C_j = number of points after j.
// A left tail (scores < a_L) is a node at a_L with A = SL; a right tail
// (scores >= a_R) a node at a_R with B = SR and count nR.
//
// gfx950 design, one 1024-thread work-group:
//   level 1 -- groups (band buckets or full-sort tiles) carry (count, first,
//     last, TA, TB); prefix and suffix anchored sums combine associatively,
//     so a work-group scan over the groups gives M at every group end and
//     the bracket certificate M(a_L) >= k >= M(a_R);
//   level 2 -- the one group whose end first drops below k is scanned
//     element by element the same way;
//   closed form -- in the located gap [x_lo, x_hi], with v = e^{(x_lo-b)/alpha},
//     w = e^{(b-x_hi)/alpha}, v w = g = e^{-(x_hi-x_lo)/alpha}, the mass is
//     A v/2 + C - B w/2 = k: a quadratic solved in the cancellation-free
//     form (log form when C = k).
// All of it in fp64.
#include "stk_common.hpp"
#include "stk_layout.hpp"
#include "stk_prof.hpp"
#include "stk_reduce.hpp"

namespace stk {

namespace {

constexpr int kT = kSelectThreads;

// An anchored exponential sum: value v anchored at point x (has = 0: empty).
struct Anch {
    double x;
    double v;
    int has;
};

// earlier e, later l (x_e <= x_l): re-anchor at l's point
__device__ __forceinline__ Anch fwd(Anch e, Anch l, double c)
{
    if (!l.has)
        return e;
    if (!e.has)
        return l;
    Anch r;
    r.x = l.x;
    r.v = l.v + exp2_nonpos((e.x - l.x) * c) * e.v;
    r.has = 1;
    return r;
}

// left l, right r (x_l <= x_r): re-anchor at l's point
__device__ __forceinline__ Anch bwd(Anch l, Anch r, double c)
{
    if (!l.has)
        return r;
    if (!r.has)
        return l;
    Anch o;
    o.x = l.x;
    o.v = l.v + exp2_nonpos((l.x - r.x) * c) * r.v;
    o.has = 1;
    return o;
}

struct ScanLds {
    double x[kT];
    double v[kT];
    int h[kT];
    unsigned long long u[kT];
};

struct ScanOut {
    Anch incl;  // over threads 0..tid (forward) or tid..nt-1 (backward)
    Anch excl;  // the same without this thread
};

__device__ __forceinline__ Anch shfl_anch(Anch a, int src_lane)
{
    Anch o;
    o.x = __shfl(a.x, src_lane, kWave);
    o.v = __shfl(a.v, src_lane, kWave);
    o.has = __shfl(a.has, src_lane, kWave);
    return o;
}

__device__ __forceinline__ Anch empty_anch()
{
    Anch a;
    a.x = 0.0;
    a.v = 0.0;
    a.has = 0;
    return a;
}

// Work-group scan of anchored sums: kForward is a prefix over threads
// 0..tid, else a suffix over tid..nt-1.  Kogge-Stone over shuffles inside
// each wave, then the wave totals (LDS) folded in order by every thread.
template <bool kForward>
__device__ ScanOut wg_scan(Anch mine, ScanLds& L, double c)
{
    constexpr int kWaves = kT / kWave;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    Anch incl = mine;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int src = kForward ? lane - off : lane + off;
        const Anch o = shfl_anch(incl, src < 0 ? 0 : (src >= kWave ? kWave - 1 : src));
        if (kForward ? lane >= off : lane + off < kWave)
            incl = kForward ? fwd(o, incl, c) : bwd(incl, o, c);
    }
    // within-wave exclusive value: the neighbour's inclusive one
    const int nb = kForward ? lane - 1 : lane + 1;
    Anch wex = shfl_anch(incl, nb < 0 ? 0 : (nb >= kWave ? kWave - 1 : nb));
    if (kForward ? lane == 0 : lane == kWave - 1)
        wex = empty_anch();
    __syncthreads();  // earlier readers of L are done
    if (kForward ? lane == kWave - 1 : lane == 0) {
        L.x[wave] = incl.x;
        L.v[wave] = incl.v;
        L.h[wave] = incl.has;
    }
    __syncthreads();
    Anch agg = empty_anch();
    if (kForward) {
        for (int w = 0; w < wave; ++w) {
            Anch t;
            t.x = L.x[w];
            t.v = L.v[w];
            t.has = L.h[w];
            agg = fwd(agg, t, c);
        }
    } else {
        for (int w = kWaves - 1; w > wave; --w) {
            Anch t;
            t.x = L.x[w];
            t.v = L.v[w];
            t.has = L.h[w];
            agg = bwd(t, agg, c);
        }
    }
    ScanOut out;
    out.incl = kForward ? fwd(agg, incl, c) : bwd(incl, agg, c);
    out.excl = kForward ? fwd(agg, wex, c) : bwd(wex, agg, c);
    return out;
}

// Inclusive prefix sum of u64 over the work-group (shuffles + wave totals).
__device__ unsigned long long wg_scan_u64(unsigned long long mine, ScanLds& L)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    unsigned long long incl = mine;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const unsigned long long o = __shfl_up(incl, off, kWave);
        if (lane >= off)
            incl += o;
    }
    __syncthreads();
    if (lane == kWave - 1)
        L.u[wave] = incl;
    __syncthreads();
    unsigned long long before = 0;
    for (int w = 0; w < wave; ++w)
        before += L.u[w];
    return before + incl;
}

__device__ int wg_max_int(int v, int* red)
{
    for (int off = 32; off > 0; off >>= 1) {
        const int o = __shfl_xor(v, off, kWave);
        v = o > v ? o : v;
    }
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0)
        red[threadIdx.x / kWave] = v;
    __syncthreads();
    int r = red[0];
    for (int w = 1; w < kT / kWave; ++w)
        r = red[w] > r ? red[w] : r;
    __syncthreads();
    return r;
}

__device__ int wg_min_int(int v, int* red)
{
    return -wg_max_int(-v, red);
}

// Mass at a point x with prefix P (anchored at x), count after C, and the
// suffix S of everything after (anchored at its first point).
__device__ __forceinline__ double mass_at(double x, double Pv, double C, Anch S, double c)
{
    double m = 0.5 * Pv + C;
    if (S.has)
        m -= 0.5 * S.v * exp2_nonpos((x - S.x) * c);
    return m;
}

// Root of A v/2 + C - B w/2 = k on [xlo, xhi] (either end may be open).
__device__ double gap_root(Anch lo, Anch hi, double C, double k, double alpha, double c)
{
    const double cc = C - k;
    if (cc == 0.0 && lo.has && hi.has)
        return 0.5 * (lo.x + hi.x) + 0.5 * alpha * log(lo.v / hi.v);
    const double g = (lo.has && hi.has) ? exp2_nonpos((lo.x - hi.x) * c) : 0.0;
    const double A = lo.has ? lo.v : 0.0;
    const double B = hi.has ? hi.v : 0.0;
    const double r = sqrt(cc * cc + A * B * g);
    if (cc > 0.0)
        return hi.x + alpha * log((cc + r) / B);
    return lo.x - alpha * log((-cc + r) / A);
}

}  // namespace

__global__ __launch_bounds__(kT) void solve_kernel(SolveArgs a)
{
    __shared__ ScanLds L;
    __shared__ int red[kT / kWave];
    __shared__ double bc_d[8];
    __shared__ unsigned long long bc_u[4];
    __shared__ int bc_i[4];

    Status* st = a.st;
    const int tid = threadIdx.x;
    const double c = a.log2e_over_alpha;
    const double k = a.k;

    // ---- route checks (tails=1: bracketed band) ---------------------------
    Anch left, right;
    left.has = 0;
    left.x = -INFINITY;
    left.v = 0.0;
    right.has = 0;
    right.x = INFINITY;
    right.v = 0.0;
    unsigned long long nR = 0;
    if (a.tails) {
        // fold the pass-1 partials (tails, counts, finiteness) into the status;
        // the band sort has pre-folded them unless the band overflowed
        const bool folded = st->nB <= (uint64_t)a.cap;
        const Pass1Partial tot = folded ? reduce_pass1(a.p1_super, kBuckets, st)
                                        : reduce_pass1(a.p1, a.p1_blocks, st);
        if (tot.nonfinite) {
            if (tid == 0)
                st->solve_state = kSolveNonfinite;
            return;
        }
        if (st->solve_state == kSolveBucketOverflow)
            return;
        if (st->nB > (uint64_t)a.cap) {
            if (tid == 0)
                st->solve_state = kSolveOverflow;
            return;
        }
        const float aL = st->aL, aR = st->aR;
        if (aL != -INFINITY) {
            left.has = 1;
            left.x = aL;
            left.v = tot.SL;
        }
        if (aR != INFINITY) {
            right.has = 1;
            right.x = aR;
            right.v = tot.SR;
        }
        nR = tot.nR;
    }

    // ---- level 1: groups ----------------------------------------------------
    const int T = a.groups;
    const int gpt = (T + kT - 1) / kT;
    const int g0 = tid * gpt < T ? tid * gpt : T;
    const int g1 = g0 + gpt < T ? g0 + gpt : T;

    Anch pre;  // this thread's groups folded forward (anchored at last hi)
    pre.has = 0;
    pre.x = 0.0;
    pre.v = 0.0;
    Anch suf;  // folded backward (anchored at first lo)
    suf.has = 0;
    suf.x = 0.0;
    suf.v = 0.0;
    unsigned long long cnt = 0;
    for (int g = g0; g < g1; ++g) {
        const GroupAgg G = a.agg[g];
        if (G.cnt == 0)
            continue;
        Anch t;
        t.has = 1;
        t.x = G.hi;
        t.v = G.TA;
        pre = fwd(pre, t, c);
        cnt += G.cnt;
    }
    for (int g = g1 - 1; g >= g0; --g) {
        const GroupAgg G = a.agg[g];
        if (G.cnt == 0)
            continue;
        Anch t;
        t.has = 1;
        t.x = G.lo;
        t.v = G.TB;
        suf = bwd(t, suf, c);
    }
    const unsigned long long cnt_incl = wg_scan_u64(cnt, L);
    if (tid == kT - 1)
        bc_u[0] = cnt_incl;  // total over groups
    const ScanOut pre_s = wg_scan<true>(pre, L, c);
    const Anch pre_before = fwd(left, pre_s.excl, c);
    if (tid == kT - 1) {
        const Anch all = fwd(left, pre_s.incl, c);
        bc_d[0] = all.x;
        bc_d[1] = all.v;
        bc_i[0] = all.has;
    }
    const ScanOut suf_s = wg_scan<false>(suf, L, c);
    const Anch suf_after = bwd(suf_s.excl, right, c);
    if (tid == 0) {
        const Anch all = bwd(suf_s.incl, right, c);
        bc_d[2] = all.x;
        bc_d[3] = all.v;
        bc_i[1] = all.has;
    }
    __syncthreads();
    const unsigned long long NG = bc_u[0];
    const unsigned long long cnt_before = cnt_incl - cnt;

    // per-group scan values: walk backward for the suffix, forward for the prefix
    {
        Anch cur = suf_after;
        for (int g = g1 - 1; g >= g0; --g) {
            const GroupAgg G = a.agg[g];
            a.scan[g].Sx = cur.has ? cur.x : INFINITY;
            a.scan[g].Sv = cur.has ? cur.v : 0.0;
            if (G.cnt) {
                Anch t;
                t.has = 1;
                t.x = G.lo;
                t.v = G.TB;
                cur = bwd(t, cur, c);
            }
        }
    }
    int cand = -1;
    {
        Anch cur = pre_before;
        unsigned long long through = cnt_before;
        for (int g = g0; g < g1; ++g) {
            const GroupAgg G = a.agg[g];
            through += G.cnt;
            const unsigned long long after = NG - through + nR;
            a.scan[g].Cafter = after;
            if (G.cnt) {
                Anch t;
                t.has = 1;
                t.x = G.hi;
                t.v = G.TA;
                cur = fwd(cur, t, c);
                a.scan[g].Pv = cur.v;
                Anch S;
                S.x = a.scan[g].Sx;
                S.v = a.scan[g].Sv;
                S.has = S.x != INFINITY;
                const double m = mass_at((double)G.hi, cur.v, (double)after, S, c);
                if (m >= k)
                    cand = g;
            }
        }
    }

    // ---- certificate of the bracket ---------------------------------------
    if (tid == 0) {
        double mL = (double)(NG + nR), mR = 0.0;
        if (a.tails) {
            Anch Sall;
            Sall.x = bc_d[2];
            Sall.v = bc_d[3];
            Sall.has = bc_i[1];
            // at a_L: left tail A = SL, everything else after it
            mL = left.has ? mass_at(left.x, left.v, (double)(NG + nR), Sall, c)
                          : (double)(NG + nR);
            // at a_R: all groups before it, right tail after it
            Anch Pall;
            Pall.x = bc_d[0];
            Pall.v = bc_d[1];
            Pall.has = bc_i[0];
            if (right.has) {
                double m = (double)nR - 0.5 * right.v;
                if (Pall.has)
                    m += 0.5 * Pall.v * exp2_nonpos((Pall.x - right.x) * c);
                mR = m;
            }
            st->massL = mL;
            st->massR = mR;
        }
        int state = kSolveOk;
        if (a.tails && left.has && !(mL >= k))
            state = kSolveRejectLow;
        else if (a.tails && right.has && !(mR <= k))
            state = kSolveRejectHigh;
        bc_i[2] = state;
    }
    __syncthreads();
    if (bc_i[2] != kSolveOk) {
        if (tid == 0)
            st->solve_state = (uint32_t)bc_i[2];
        return;
    }

    // ---- locate the group -----------------------------------------------------
    const int tstar = wg_max_int(cand, red);
    int unext = T;
    for (int g = g0; g < g1; ++g) {
        if (g > tstar && a.agg[g].cnt != 0) {
            unext = g;
            break;
        }
    }
    const int u = wg_min_int(unext, red);

    // lower end of the located interval: the node at group t*'s end (or a_L)
    Anch lo_node = left;
    if (tstar >= 0) {
        lo_node.has = 1;
        lo_node.x = a.agg[tstar].hi;
        lo_node.v = a.scan[tstar].Pv;
    }

    if (u >= T) {
        // root between the last group and the right node
        if (tid == 0) {
            const double b = gap_root(lo_node, right, (double)nR, k, a.alpha, c);
            *a.out_b = b;
            st->b = b;
            st->solve_state = isfinite(b) ? kSolveOk : kSolveRejectHigh;
        }
        return;
    }
    const GroupAgg U = a.agg[u];
    Anch Su;
    Su.x = a.scan[u].Sx;
    Su.v = a.scan[u].Sv;
    Su.has = Su.x != INFINITY;
    const unsigned long long Cu = a.scan[u].Cafter;
    if (U.lo == U.hi) {
        // every value of the group is equal: the root lies before it
        if (tid == 0) {
            Anch t;
            t.has = 1;
            t.x = U.lo;
            t.v = U.TB;
            const Anch hi_node = bwd(t, Su, c);
            const double b = gap_root(lo_node, hi_node, (double)(U.cnt + Cu), k, a.alpha, c);
            *a.out_b = b;
            st->b = b;
            st->solve_state = isfinite(b) ? kSolveOk : kSolveRejectHigh;
        }
        return;
    }

    // ---- level 2: elements of group u -------------------------------------------
    // group sizes are <= kBucketCap (band buckets that are not all-equal) or
    // kTile (full-sort tiles), so each thread holds at most kEpt elements
    constexpr int kEpt = 8;
    static_assert(kBucketCap <= kEpt * kT && kTile <= kEpt * kT, "group too large for level 2");
    const int cntu = (int)U.cnt;
    const int ept = (cntu + kT - 1) / kT;
    const int e0 = tid * ept < cntu ? tid * ept : cntu;
    const int e1 = e0 + ept < cntu ? e0 + ept : cntu;
    float xs[kEpt];
    double Av[kEpt];  // prefix within this thread's elements, anchored at xs[i]
    double Bv[kEpt];  // suffix within this thread's elements, anchored at xs[i]
    const float* xg = a.sorted + U.start;
#pragma unroll
    for (int i = 0; i < kEpt; ++i)
        xs[i] = (e0 + i < e1) ? xg[e0 + i] : 0.f;
    Anch lp;
    lp.has = 0;
    lp.x = 0.0;
    lp.v = 0.0;
#pragma unroll
    for (int i = 0; i < kEpt; ++i) {
        if (e0 + i < e1) {
            Anch t;
            t.has = 1;
            t.x = xs[i];
            t.v = 1.0;
            lp = fwd(lp, t, c);
        }
        Av[i] = lp.v;
    }
    Anch ls;
    ls.has = 0;
    ls.x = 0.0;
    ls.v = 0.0;
#pragma unroll
    for (int i = kEpt - 1; i >= 0; --i) {
        if (e0 + i < e1) {
            Anch t;
            t.has = 1;
            t.x = xs[i];
            t.v = 1.0;
            ls = bwd(t, ls, c);
        }
        Bv[i] = ls.v;
    }
    const Anch ex_pre = fwd(lo_node, wg_scan<true>(lp, L, c).excl, c);
    const Anch ex_suf = bwd(wg_scan<false>(ls, L, c).excl, Su, c);

    int jc = -1;
#pragma unroll
    for (int i = 0; i < kEpt; ++i) {
        const int j = e0 + i;
        if (j < e1) {
            Anch Ai;
            Ai.has = 1;
            Ai.x = xs[i];
            Ai.v = Av[i];
            const Anch Aj = fwd(ex_pre, Ai, c);
            Anch Bn = ex_suf;
            if (i + 1 < kEpt && j + 1 < e1) {
                Anch Bi;
                Bi.has = 1;
                Bi.x = xs[i + 1];
                Bi.v = Bv[i + 1];
                Bn = bwd(Bi, ex_suf, c);
            }
            const double C = (double)(cntu - 1 - j) + (double)Cu;
            const double m = mass_at((double)xs[i], Aj.v, C, Bn, c);
            if (m >= k)
                jc = j;
        }
    }
    const int jstar = wg_max_int(jc, red);
    // owners publish the two ends of the gap
    if (jstar < 0 && tid == 0) {
        bc_d[0] = lo_node.x;
        bc_d[1] = lo_node.v;
        bc_i[0] = lo_node.has;
    }
#pragma unroll
    for (int i = 0; i < kEpt; ++i) {
        const int j = e0 + i;
        if (j < e1 && j == jstar) {
            Anch Ai;
            Ai.has = 1;
            Ai.x = xs[i];
            Ai.v = Av[i];
            const Anch Aj = fwd(ex_pre, Ai, c);
            bc_d[0] = Aj.x;
            bc_d[1] = Aj.v;
            bc_i[0] = 1;
        }
        if (j < e1 && j == jstar + 1) {
            Anch Bi;
            Bi.has = 1;
            Bi.x = xs[i];
            Bi.v = Bv[i];
            const Anch Bj = bwd(Bi, ex_suf, c);
            bc_d[2] = Bj.x;
            bc_d[3] = Bj.v;
            bc_i[1] = 1;
        }
    }
    if (jstar + 1 >= cntu && tid == 0) {
        bc_d[2] = Su.x;
        bc_d[3] = Su.v;
        bc_i[1] = Su.has;
    }
    __syncthreads();
    if (tid == 0) {
        Anch lo, hi;
        lo.x = bc_d[0];
        lo.v = bc_d[1];
        lo.has = bc_i[0];
        hi.x = bc_d[2];
        hi.v = bc_d[3];
        hi.has = bc_i[1];
        const double C = (jstar + 1 < cntu) ? (double)(cntu - 1 - jstar) + (double)Cu : (double)Cu;
        const double b = gap_root(lo, hi, C, k, a.alpha, c);
        *a.out_b = b;
        st->b = b;
        st->solve_state = isfinite(b) ? kSolveOk : kSolveRejectHigh;
    }
}

hipError_t launch_solve(const SolveArgs& a, hipStream_t stream)
{
    STK_LAUNCH(kKSolve, stream, solve_kernel, dim3(1), dim3(kT), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Full-sort route: summaries of fixed tiles of the sorted keys.  The keys are
// turned back into fp32 values in place, so the solve reads one float array.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSortThreads) void tile_agg_kernel(TileArgs a)
{
    __shared__ double red[2][kSortThreads / kWave];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int64_t i0 = (int64_t)t * kTile;
    const int64_t i1 = i0 + kTile < a.n ? i0 + kTile : a.n;
    const uint32_t cnt = (uint32_t)(i1 - i0);
    const float lo = key_to_float(a.keys[i0] + a.key_min);
    const float hi = key_to_float(a.keys[i1 - 1] + a.key_min);
    __syncthreads();  // lo/hi read by all before anyone rewrites i0 / i1-1
    const double c = a.log2e_over_alpha;
    const double dlo = lo, dhi = hi;
    double TA = 0.0, TB = 0.0;
    for (int64_t i = i0 + tid; i < i1; i += kSortThreads) {
        const float v = key_to_float(a.keys[i] + a.key_min);
        a.keys[i] = __float_as_uint(v);
        TA += exp2_nonpos(((double)v - dhi) * c);
        TB += exp2_nonpos((dlo - (double)v) * c);
    }
    TA = wave_sum(TA);
    TB = wave_sum(TB);
    if (lane == 0) {
        red[0][wave] = TA;
        red[1][wave] = TB;
    }
    __syncthreads();
    if (tid == 0) {
        GroupAgg g;
        g.TA = 0.0;
        g.TB = 0.0;
        for (int w = 0; w < kSortThreads / kWave; ++w) {
            g.TA += red[0][w];
            g.TB += red[1][w];
        }
        g.lo = lo;
        g.hi = hi;
        g.cnt = cnt;
        g.start = (uint32_t)i0;
        a.agg[t] = g;
    }
}

hipError_t launch_tile_aggregates(const TileArgs& a, hipStream_t stream)
{
    STK_LAUNCH(kKTileAgg, stream, tile_agg_kernel, dim3(a.n_tiles), dim3(kSortThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace stk
