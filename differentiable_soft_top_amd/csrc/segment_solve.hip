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
// gfx950 design, one 512-thread work-group:
//   level 1 -- groups (band buckets or full-sort tiles) carry (count, first,
//     last, TA, TB); prefix and suffix anchored sums combine associatively,
//     so a work-group scan over the groups gives M at every group end and
//     the bracket certificate M(a_L) >= k >= M(a_R);
//   level 2 -- the one group whose end first drops below k is sorted in LDS
//     (band buckets arrive unordered; full-sort tiles arrive sorted) and
//     scanned element by element the same way;
//   direct -- a band small enough for one LDS sort skips the buckets: it is
//     sorted and scanned whole at level 2, and the certificate comes from
//     that scan's totals;
//   closed form -- in the located gap [x_lo, x_hi], with v = e^{(x_lo-b)/alpha},
//     w = e^{(b-x_hi)/alpha}, v w = g = e^{-(x_hi-x_lo)/alpha}, the mass is
//     A v/2 + C - B w/2 = k: a quadratic solved in the cancellation-free
//     form (log form when C = k).
// All of it in fp64.
#include "stk_common.hpp"
#include "stk_layout.hpp"
#include "stk_prof.hpp"
#include "stk_reduce.hpp"
#include "stk_scan.hpp"

namespace stk {

namespace {

constexpr int kST = kSolveThreads;       // threads of the solve work-group
constexpr int kSW = kST / kWave;         // its waves
static_assert(kTile <= kBucketCap, "full-sort tiles must fit the level-2 buffers");
static_assert(kBuckets % kST == 0, "pass-1 super partials per thread");

// ---------------------------------------------------------------------------
// Reference-point sums.  When every point of a solve lies within kRefSpan
// (in units of alpha / log2 e) of a reference r, the anchored sums of the
// full-sort solver are ratios of plain sums: with E(x) = 2^{(x - r) c}
// (c = log2 e / alpha),
//   sum_{i <= j} e^{(x_i - x_j)/alpha} = (sum_{i <= j} E_i) / E_j,
//   sum_{i >  j} e^{-(x_i - x_j)/alpha} = E_j * sum_{i > j} 1/E_i,
// and every E and 1/E is a normal fp64 number.  The work-group scans then
// carry fp64 additions instead of an exponential per combination, and each
// point costs one exponential, evaluated independently rather than along a
// dependency chain.  All sums are of positive terms (relative error ~1e-16
// times the scan depth), as accurate as the anchored form.  A bracket end at
// infinity, or a wider span, keeps the anchored form.
// ---------------------------------------------------------------------------
constexpr double kRefSpan = 1800.0;

// 2^y for |y| <= 1022: the series of exp2_nonpos without its clamp to y <= 0.
__device__ __forceinline__ double exp2_ref(double y)
{
    const double j = __builtin_rint(y);
    const double t = (y - j) * kLn2;
    double p = 2.08767569878681e-09;
    p = fma(p, t, 2.505210838544172e-08);
    p = fma(p, t, 2.755731922398589e-07);
    p = fma(p, t, 2.7557319223985893e-06);
    p = fma(p, t, 2.48015873015873e-05);
    p = fma(p, t, 0.0001984126984126984);
    p = fma(p, t, 0.001388888888888889);
    p = fma(p, t, 0.008333333333333333);
    p = fma(p, t, 0.041666666666666664);
    p = fma(p, t, 0.16666666666666666);
    p = fma(p, t, 0.5);
    p = fma(p, t, 1.0);
    p = fma(p, t, 1.0);
    return ldexp(p, (int)j);
}

// Exclusive work-group scans of a pair of fp64 sums and a count: the
// prefix of p over earlier threads, the suffix of s over later threads,
// the prefix of the count, and the three totals.  Exclusive values come
// from shifting the inclusive ones (no subtraction), so a small sum next to
// a large one keeps its relative accuracy.
struct RefScan {
    double p_before, s_after, p_all, s_all;
    uint32_t c_before, c_all;
};

template <int kSWn>
__device__ __forceinline__ RefScan ref_scan_publish(double p, double s, uint32_t cnt, WaveTot* wt, RefScan* part)
{
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    double pi = p, si = s;
    uint32_t ci = cnt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double op = __shfl_up(pi, off, kWave);
        const double os = __shfl_down(si, off, kWave);
        const uint32_t oc = __shfl_up(ci, off, kWave);
        if (lane >= off) {
            pi += op;
            ci += oc;
        }
        if (lane + off < kWave)
            si += os;
    }
    RefScan r;
    r.p_before = __shfl_up(pi, 1, kWave);
    r.c_before = __shfl_up(ci, 1, kWave);
    r.s_after = __shfl_down(si, 1, kWave);
    if (lane == 0) {
        r.p_before = 0.0;
        r.c_before = 0u;
    }
    if (lane == kWave - 1)
        r.s_after = 0.0;
    if (lane == kWave - 1) {
        wt[wave].pv = pi;
        wt[wave].cnt = ci;
    }
    if (lane == 0)
        wt[wave].sv = si;
    *part = r;
    return r;
}

// after the barrier that follows ref_scan_publish
template <int kSWn>
__device__ __forceinline__ RefScan ref_scan_finish(const WaveTot* wt, const RefScan& part)
{
    const int wave = threadIdx.x / kWave;
    RefScan r = part;
    double pb = 0.0, sa = 0.0, pall = 0.0, sall = 0.0;
    uint32_t cb = 0u, call = 0u;
    for (int w = 0; w < kSWn; ++w) {
        if (w < wave) {
            pb += wt[w].pv;
            cb += wt[w].cnt;
        }
        pall += wt[w].pv;
        call += wt[w].cnt;
    }
    for (int w = kSWn - 1; w >= 0; --w) {
        if (w > wave)
            sa += wt[w].sv;
        sall += wt[w].sv;
    }
    r.p_before += pb;
    r.c_before += cb;
    r.s_after += sa;
    r.p_all = pall;
    r.s_all = sall;
    r.c_all = call;
    return r;
}

// Load cnt values (R per thread), sort into keys[0 .. cnt).  Bucket sort
// first (band values are spread evenly over a narrow range); if a bucket
// overflows its register network, the values are loaded again and sorted by
// a bitonic network, padded with +inf to kST * R.  spare: LDS, kST * R words.
template <int R>
__device__ __forceinline__ void load_keys(const float* x, int cnt, uint32_t (&v)[R])
{
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = threadIdx.x * R + r;
        v[r] = i < cnt ? float_to_key(x[i]) : 0xFFFFFFFFu;
    }
}

template <int R>
__device__ __forceinline__ void sort_group_into(const float* x, int cnt, uint32_t* keys, uint32_t* spare)
{
    {
        uint32_t v[R];
        load_keys<R>(x, cnt, v);
        if (block_bucket_sort<kST, R>(v, cnt, keys, spare))
            return;
    }
    uint32_t v[R];
    load_keys<R>(x, cnt, v);
    block_bitonic_regs<kST, R>(v, keys, spare);
    __syncthreads();  // the last LDS stage's reads are done
#pragma unroll
    for (int r = 0; r < R; ++r)
        keys[threadIdx.x * R + r] = v[r];
}

// What a thread publishes about the groups it owns: the last one whose end
// carries mass >= k (lo side of the root) and the first non-empty one whose
// end carries less (the group that holds the root).
struct RowHi {
    GroupAgg g;
    double Sv;                     // suffix of everything after the group
    float Sx;
    uint32_t Cafter;               // scores after the group (right tail included)
};

struct SolveLds {
    WaveTot wt[kSW];
    double pd[2][kSW];
    unsigned long long pu[2][kSW];
    uint32_t pnf[kSW];
    float pf[4][kSW];
    int imax[kSW], imin[kSW];
    Anch lo[kST];
    RowHi hi[kST];
    uint32_t keys[kBucketCap];
    double bv[kBucketCap];
};

__device__ __forceinline__ void block_max_min(int vmax, int vmin, SolveLds& L, int* omax, int* omin)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const int a = __shfl_xor(vmax, off, kWave);
        const int b = __shfl_xor(vmin, off, kWave);
        vmax = a > vmax ? a : vmax;
        vmin = b < vmin ? b : vmin;
    }
    if (lane_id() == 0) {
        L.imax[threadIdx.x / kWave] = vmax;
        L.imin[threadIdx.x / kWave] = vmin;
    }
    __syncthreads();
    int M = L.imax[0], m = L.imin[0];
    for (int w = 1; w < kSW; ++w) {
        M = L.imax[w] > M ? L.imax[w] : M;
        m = L.imin[w] < m ? L.imin[w] : m;
    }
    *omax = M;
    *omin = m;
}

__device__ __forceinline__ void finish(const SolveArgs& a, double b)
{
    *a.out_b = b;
    a.st->b = b;
    a.st->solve_state = isfinite(b) ? kSolveOk : kSolveRejectHigh;
}

// Level 2: cnt values at x (cnt >= 1 unless `certify`), sorted into LDS
// unless they arrive sorted, scanned element by element between lo_node
// (everything before them) and Su / Cu (the suffix and the count of
// everything after them); the last breakpoint with mass >= k is located and
// the closed form applied in the gap after it.  With `certify` the values
// are the whole band, lo_node / Su the tail nodes and Cu the right-tail
// count: the bracket certificate is then taken from the scan's totals first.
struct Level2Job {
    const float* xg;
    int cntu;
    bool unsorted, certify, hasL, hasR;
    Anch lo_node, Su;
    uint32_t Cu;
};

// Whether level 2 can use reference-point sums: the end nodes that carry
// weight and the group's values within kRefSpan; *ref gets the reference.
__device__ __forceinline__ bool level2_ref_ok(const Level2Job& job, const SolveLds& L, double c, double* ref)
{
    if (job.cntu < 1)
        return false;
    double lo = key_to_float(L.keys[0]);
    double hi = key_to_float(L.keys[job.cntu - 1]);
    if (job.lo_node.v > 0.0)
        lo = fmin(lo, (double)job.lo_node.x);
    if (job.Su.v > 0.0)
        hi = fmax(hi, (double)job.Su.x);
    if (!(lo > -INFINITY && hi < INFINITY) || !((hi - lo) * c <= kRefSpan))
        return false;
    *ref = 0.5 * (lo + hi);
    return true;
}

// Level 2 with reference-point sums (the same breakpoint masses, the same
// last breakpoint with mass >= k and the same closed form as `level2`).
__device__ __forceinline__ void level2_ref(const SolveArgs& a, SolveLds& L, const Level2Job& job, double ref)
{
    const int cntu = job.cntu;
    const Anch lo_node = job.lo_node, Su = job.Su;
    const uint32_t Cu = job.Cu;
    Status* st = a.st;
    const int tid = threadIdx.x;
    const double c = a.log2e_over_alpha;
    const double k = a.k;
    const int ept = (cntu + kST - 1) / kST;
    const int e0 = tid * ept < cntu ? tid * ept : cntu;
    const int e1 = e0 + ept < cntu ? e0 + ept : cntu;
    // this thread's points: E in the prefix, 1/E in a suffix kept per point
    double pe = 0.0, sf = 0.0;
    for (int j = e1 - 1; j >= e0; --j) {
        const double E = exp2_ref(((double)key_to_float(L.keys[j]) - ref) * c);
        pe += E;
        sf += 1.0 / E;
        L.bv[j] = sf;
    }
    RefScan part;
    ref_scan_publish<kSW>(pe, sf, 0u, L.wt, &part);
    __syncthreads();
    const RefScan rs = ref_scan_finish<kSW>(L.wt, part);
    // the end nodes in reference units
    const double Pbase = lo_node.v > 0.0 ? lo_node.v * exp2_ref(((double)lo_node.x - ref) * c) : 0.0;
    const double Sbase = Su.v > 0.0 ? Su.v * exp2_ref(-((double)Su.x - ref) * c) : 0.0;

    if (job.certify) {
        // M(a_L) >= k >= M(a_R) from the band's totals and the tails
        const double all = (double)cntu + (double)Cu;
        const double mL = job.hasL ? 0.5 * lo_node.v + all -
                                         0.5 * exp2_ref(((double)lo_node.x - ref) * c) * (rs.s_all + Sbase)
                                   : all;
        double mR = 0.0;
        if (job.hasR)
            mR = (double)Cu - 0.5 * Su.v + 0.5 * exp2_ref(-((double)Su.x - ref) * c) * (rs.p_all + Pbase);
        if (tid == 0) {
            st->massL = mL;
            st->massR = mR;
        }
        const bool rejL = job.hasL && !(mL >= k);
        const bool rejR = !rejL && job.hasR && !(mR <= k);
        if (rejL || rejR) {
            if (tid == 0)
                st->solve_state = rejL ? kSolveRejectLow : kSolveRejectHigh;
            return;
        }
    }

    // breakpoint masses: M(x_j) = A_j / 2 + C_j - T_j / 2 with
    // A_j = (Pbase + sum_{i<=j} E_i) / E_j and T_j = E_j (sum_{i>j} 1/E_i + Sbase)
    int jc = -1;
    double jA = 0.0, jS = 0.0;
    double P = Pbase + rs.p_before;
    for (int j = e0; j < e1; ++j) {
        const double E = exp2_ref(((double)key_to_float(L.keys[j]) - ref) * c);
        P += E;
        const double Safter = rs.s_after + (j + 1 < e1 ? L.bv[j + 1] : 0.0) + Sbase;
        const double m = 0.5 * (P / E) + ((double)(cntu - 1 - j) + (double)Cu) - 0.5 * (E * Safter);
        if (m >= k) {
            jc = j;
            jA = P / E;
            jS = Safter;
        }
    }
    int jstar, unused;
    block_max_min(jc, 0, L, &jstar, &unused);  // [1]
    if (jstar >= 0) {
        if (jc == jstar) {
            // the gap after x_j*: its prefix anchored at x_j*, its suffix at
            // the next point (or the end node)
            const float xn = jstar + 1 < cntu ? key_to_float(L.keys[jstar + 1]) : Su.x;
            const Anch hi = jS > 0.0 ? node(xn, jS * exp2_ref(((double)xn - ref) * c)) : empty_suf();
            finish(a, gap_root(node(key_to_float(L.keys[jstar]), jA), hi, (double)(cntu - 1 - jstar) + (double)Cu, k,
                               a.alpha, c));
        }
    } else if (tid == 0) {
        // the root lies before the first point
        const float x0 = key_to_float(L.keys[0]);
        const Anch B0 = node(x0, (rs.s_all + Sbase) * exp2_ref(((double)x0 - ref) * c));
        finish(a, gap_root(lo_node, B0, (double)cntu + (double)Cu, k, a.alpha, c));
    }
}

__device__ __forceinline__ void level2(const SolveArgs& a, SolveLds& L, const Level2Job& job)
{
    const float* xg = job.xg;
    const int cntu = job.cntu;
    const Anch lo_node = job.lo_node, Su = job.Su;
    const uint32_t Cu = job.Cu;
    const bool certify = job.certify, hasL = job.hasL, hasR = job.hasR;
    Status* st = a.st;
    const int tid = threadIdx.x;
    const double c = a.log2e_over_alpha;
    const double k = a.k;
    if (job.unsorted) {
        uint32_t* spare = reinterpret_cast<uint32_t*>(L.bv);
        if (cntu <= kST)
            sort_group_into<1>(xg, cntu, L.keys, spare);
        else if (cntu <= 2 * kST)
            sort_group_into<2>(xg, cntu, L.keys, spare);
        else if (cntu <= 4 * kST)
            sort_group_into<4>(xg, cntu, L.keys, spare);
        else if (cntu <= 8 * kST)
            sort_group_into<8>(xg, cntu, L.keys, spare);
        else
            sort_group_into<16>(xg, cntu, L.keys, spare);
    } else {
        for (int i = tid; i < cntu; i += kST)
            L.keys[i] = float_to_key(xg[i]);
    }
    __syncthreads();
    double ref = 0.0;
    if (level2_ref_ok(job, L, c, &ref)) {
        level2_ref(a, L, job, ref);
        return;
    }
    const int ept = (cntu + kST - 1) / kST;
    const int e0 = tid * ept < cntu ? tid * ept : cntu;
    const int e1 = e0 + ept < cntu ? e0 + ept : cntu;
    // this thread's elements: the backward chain (suffix within the thread,
    // anchored at each element) kept in LDS, the forward fold in registers
    Anch ls = empty_suf();
    for (int j = e1 - 1; j >= e0; --j) {
        ls = bwd(node(key_to_float(L.keys[j]), 1.0), ls, c);
        L.bv[j] = ls.v;
    }
    Anch lp = empty_pre();
    for (int j = e0; j < e1; ++j)
        lp = fwd(lp, node(key_to_float(L.keys[j]), 1.0), c);
    const Scan2Part part2 = scan2_publish(lp, ls, 0u, c, L.wt);
    __syncthreads();  // [1]
    const Scan2 s2 = scan2_finish<kSW>(L.wt, part2, c);
    const Anch ex_pre = fwd(lo_node, s2.pre_before, c);
    const Anch ex_suf = bwd(s2.suf_after, Su, c);

    if (certify) {
        // M(a_L) >= k >= M(a_R) from the band's totals and the tails
        const double all = (double)cntu + (double)Cu;
        const Anch Sall = bwd(s2.suf_all, Su, c);
        const double mL = hasL ? mass_at(lo_node.x, lo_node.v, all, Sall, c) : all;
        double mR = 0.0;
        if (hasR) {
            const Anch Pall = fwd(lo_node, s2.pre_all, c);
            mR = (double)Cu - 0.5 * Su.v + 0.5 * Pall.v * exp2_nonpos(((double)Pall.x - (double)Su.x) * c);
        }
        if (tid == 0) {
            st->massL = mL;
            st->massR = mR;
        }
        const bool rejL = hasL && !(mL >= k);
        const bool rejR = !rejL && hasR && !(mR <= k);
        if (rejL || rejR) {
            if (tid == 0)
                st->solve_state = rejL ? kSolveRejectLow : kSolveRejectHigh;
            return;
        }
        if (cntu == 0) {
            // empty band: the root lies between the two tail nodes
            if (tid == 0)
                finish(a, gap_root(lo_node, Su, (double)Cu, k, a.alpha, c));
            return;
        }
    }

    // breakpoint masses: A_j walks forward from everything before, B_{j+1}
    // is the stored chain re-anchored onto everything after
    int jc = -1;
    Anch jlo = empty_pre(), jhi = empty_suf();
    Anch A = ex_pre;
    for (int j = e0; j < e1; ++j) {
        const float xj = key_to_float(L.keys[j]);
        A = fwd(A, node(xj, 1.0), c);
        const Anch Bn = j + 1 < e1 ? bwd(node(key_to_float(L.keys[j + 1]), L.bv[j + 1]), ex_suf, c) : ex_suf;
        if (mass_at(xj, A.v, (double)(cntu - 1 - j) + (double)Cu, Bn, c) >= k) {
            jc = j;
            jlo = A;
            jhi = Bn;
        }
    }
    int jstar, unused;
    block_max_min(jc, 0, L, &jstar, &unused);  // [1]
    if (jstar >= 0) {
        if (jc == jstar)
            finish(a, gap_root(jlo, jhi, (double)(cntu - 1 - jstar) + (double)Cu, k, a.alpha, c));
    } else if (tid == 0) {
        // the root lies before the first point
        const Anch B0 = bwd(node(key_to_float(L.keys[0]), L.bv[0]), ex_suf, c);
        finish(a, gap_root(lo_node, B0, (double)cntu + (double)Cu, k, a.alpha, c));
    }
}

}  // namespace

// Level 1 of the bucket route in reference-point sums (one group per
// thread; the bracket ends finite and within kRefSpan): the bracket
// certificate, the mass at every group end, the two groups around the
// root, then the level-2 job, as in solve_levels.  left / right: the tail
// nodes; rs: the scans of this thread's group terms.
__device__ __forceinline__ bool solve_level1_ref(const SolveArgs& a, SolveLds& L, Level2Job& job, const GroupAgg& mine, int g0,
                                 double ref, double Eh, const RefScan& rs, Anch left, Anch right, uint64_t nR)
{
    Status* st = a.st;
    const int tid = threadIdx.x;
    const double c = a.log2e_over_alpha;
    const double k = a.k;
    const int T = a.groups;
    const uint32_t NG = rs.c_all;
    const double EaL = exp2_ref(((double)left.x - ref) * c);
    const double FaR = exp2_ref(-((double)right.x - ref) * c);
    const double Pbase = left.v * EaL;
    const double Sbase = right.v * FaR;

    // ---- bracket certificate (every thread, same values) ---------------------------
    const double mL = 0.5 * left.v + ((double)NG + (double)nR) - 0.5 * EaL * (rs.s_all + Sbase);
    const double mR = (double)nR - 0.5 * right.v + 0.5 * FaR * (rs.p_all + Pbase);
    if (tid == 0) {
        st->massL = mL;
        st->massR = mR;
    }
    const bool rejL = !(mL >= k);
    const bool rejR = !rejL && !(mR <= k);
    if (rejL || rejR) {
        if (tid == 0)
            st->solve_state = rejL ? kSolveRejectLow : kSolveRejectHigh;
        return false;
    }

    // ---- masses at the group ends; the two groups around the root ----------------------
    // after this group: its suffix anchored at the group's end (every later
    // point lies at or above it)
    const double s_after = rs.s_after + Sbase;
    const uint32_t after = NG - (rs.c_before + mine.cnt) + (uint32_t)nR;
    const Anch suf_here = s_after > 0.0 ? node(mine.hi, s_after * Eh) : empty_suf();
    int tc = -1, uc = T;
    if (g0 < T && mine.cnt) {
        const double A = (Pbase + rs.p_before + mine.TA * Eh) / Eh;
        const double m = 0.5 * A + (double)after - 0.5 * (Eh * s_after);
        if (m >= k) {
            tc = g0;
            L.lo[tid] = node(mine.hi, A);
        } else {
            uc = g0;
            L.hi[tid].g = mine;
            L.hi[tid].Sx = suf_here.x;
            L.hi[tid].Sv = suf_here.v;
            L.hi[tid].Cafter = after;
        }
    }
    int tstar, u;
    block_max_min(tc, uc, L, &tstar, &u);  // [1]
    if (u < tstar) {
        // rounding broke the monotone order of the group-end masses: take
        // the first non-empty group after t* instead
        __syncthreads();
        int mine_u = T;
        if (g0 < T && g0 > tstar && mine.cnt) {
            mine_u = g0;
            L.hi[tid].g = mine;
            L.hi[tid].Sx = suf_here.x;
            L.hi[tid].Sv = suf_here.v;
            L.hi[tid].Cafter = after;
        }
        int dummy;
        block_max_min(-1, mine_u, L, &dummy, &u);
    }
    Anch lo_node = left;
    if (tstar >= 0)
        lo_node = L.lo[tstar];
    if (u >= T) {
        // root between the last group and the right node
        if (tid == 0)
            finish(a, gap_root(lo_node, right, (double)nR, k, a.alpha, c));
        return false;
    }
    const RowHi Ur = L.hi[u];
    const GroupAgg U = Ur.g;
    const Anch Su = node(Ur.Sx, Ur.Sv);
    const uint32_t Cu = Ur.Cafter;
    if (U.lo == U.hi) {
        // every value of the group is equal: the root lies before it
        if (tid == 0)
            finish(a, gap_root(lo_node, bwd(node(U.lo, U.TB), Su, c), (double)U.cnt + (double)Cu, k, a.alpha, c));
        return false;
    }
    const int cntu = (int)U.cnt;
    if (cntu > kBucketCap) {
        if (tid == 0)
            st->solve_state = kSolveBucketOverflow;
        return false;
    }
    job.xg = a.sorted + U.start;
    job.cntu = cntu;
    job.unsorted = true;
    job.certify = false;
    job.hasL = false;
    job.hasR = false;
    job.lo_node = lo_node;
    job.Su = Su;
    job.Cu = Cu;
    return true;
}

// One work-group.  Phases (barriers in brackets):
//   1. fold the pass-1 partials; per-thread level-1 values; wave scans  [1]
//   2. per-group masses, bracket certificate, the two groups around the
//      root published to LDS                                            [1]
//   (a directly sorted band skips 1's scans and 2: it goes to level 2 whole)
//   3. level 2 (`level2`): the located group into LDS, sorted unless it
//      comes from the full sort                                         [few]
//   4. level-2 scans, breakpoint masses                                 [1]
//   5. the last breakpoint with mass >= k; its owner applies the closed
//      form                                                             [1]
// Returns whether level 2 is needed (false: b or a rejection is recorded).
__device__ __forceinline__ bool solve_levels(const SolveArgs& a, SolveLds& L, Level2Job& job)
{
    Status* st = a.st;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const double c = a.log2e_over_alpha;
    const double k = a.k;

    // ---- loads issued up front ----------------------------------------------
    const int T = a.groups;
    const int gpt = (T + kST - 1) / kST;
    const int g0 = tid * gpt < T ? tid * gpt : T;
    const int g1 = g0 + gpt < T ? g0 + gpt : T;
    GroupAgg mine;
    mine.cnt = 0;
    if (gpt == 1 && g0 < T)
        mine = a.agg[g0];
    const uint64_t nB = a.tails ? st->nB : 0;
    const float aL = a.tails ? st->aL : -INFINITY;
    const float aR = a.tails ? st->aR : INFINITY;

    // pass-1 totals (tails, counts, finiteness): the band sort pre-folded
    // them into kBuckets partials unless the band overflowed; those are read
    // speculatively, together with the band count that says whether they hold
    double SL = 0.0, SR = 0.0;
    unsigned long long nL = 0, nR = 0;
    uint32_t nf = 0;
    float bmin = INFINITY, bmax = -INFINITY, smin = INFINITY, smax = -INFINITY;
    auto add = [&](const Pass1Partial& p) {
        SL += p.SL;
        SR += p.SR;
        nL += p.nL;
        nR += p.nR;
        nf |= p.nonfinite;
        bmin = fminf(bmin, p.bmin);
        bmax = fmaxf(bmax, p.bmax);
        smin = fminf(smin, p.smin);
        smax = fmaxf(smax, p.smax);
    };
    if (a.tails) {
        constexpr int kSp = kBuckets / kST;
        Pass1Partial sp[kSp];
        if (!a.direct) {
#pragma unroll
            for (int r = 0; r < kSp; ++r)
                sp[r] = a.p1_super[r * kST + tid];
        }
        if (!a.direct && nB <= (uint64_t)a.cap) {
#pragma unroll
            for (int r = 0; r < kSp; ++r)
                add(sp[r]);
        } else {
            for (int i = tid; i < a.p1_blocks; i += kST)
                add(a.p1[i]);
        }
    }
    SL = wave_sum(SL);
    SR = wave_sum(SR);
    nL = wave_sum_u64(nL);
    nR = wave_sum_u64(nR);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        nf |= __shfl_xor(nf, off, kWave);
    bmin = wave_min(bmin);
    bmax = wave_max(bmax);
    smin = wave_min(smin);
    smax = wave_max(smax);
    if (lane == 0) {
        L.pd[0][wave] = SL;
        L.pd[1][wave] = SR;
        L.pu[0][wave] = nL;
        L.pu[1][wave] = nR;
        L.pnf[wave] = nf;
        L.pf[0][wave] = bmin;
        L.pf[1][wave] = bmax;
        L.pf[2][wave] = smin;
        L.pf[3][wave] = smax;
    }

    // ---- level 1: this thread's groups folded, then the work-group scans ------------
    Anch pre = empty_pre(), suf = empty_suf();
    uint32_t cnt = 0;
    if (gpt == 1) {
        if (g0 < T && mine.cnt) {
            pre = node(mine.hi, mine.TA);
            suf = node(mine.lo, mine.TB);
            cnt = mine.cnt;
        }
    } else {
        for (int g = g0; g < g1; ++g) {
            const GroupAgg G = a.agg[g];
            if (G.cnt) {
                pre = fwd(pre, node(G.hi, G.TA), c);
                cnt += G.cnt;
            }
        }
        for (int g = g1 - 1; g >= g0; --g) {
            const GroupAgg G = a.agg[g];
            if (G.cnt)
                suf = bwd(node(G.lo, G.TB), suf, c);
        }
    }
    // bucket route with a finite bracket no wider than kRefSpan: level 1 in
    // reference-point sums (reference at the bracket's midpoint)
    const bool use_ref = a.tails && !a.direct && gpt == 1 && aL > -INFINITY && aR < INFINITY &&
                         ((double)aR - (double)aL) * c <= kRefSpan;
    const double ref = use_ref ? 0.5 * ((double)aL + (double)aR) : 0.0;
    double Eh = 1.0;  // E at this thread's group end
    RefScan rpart;
    Scan2Part part1;
    if (use_ref) {
        double pg = 0.0, sg = 0.0;
        if (g0 < T && mine.cnt) {
            Eh = exp2_ref(((double)mine.hi - ref) * c);
            pg = mine.TA * Eh;
            sg = mine.TB * exp2_ref(-((double)mine.lo - ref) * c);
        }
        ref_scan_publish<kSW>(pg, sg, cnt, L.wt, &rpart);
    } else if (!a.direct) {
        part1 = scan2_publish(pre, suf, cnt, c, L.wt);
    }
    __syncthreads();  // [1]

    // every thread folds the wave values in the same order
    SL = SR = 0.0;
    nL = nR = 0;
    nf = 0;
    for (int w = 0; w < kSW; ++w) {
        SL += L.pd[0][w];
        SR += L.pd[1][w];
        nL += L.pu[0][w];
        nR += L.pu[1][w];
        nf |= L.pnf[w];
    }
    if (a.tails && tid == 0) {
        float f0 = INFINITY, f1 = -INFINITY, f2 = INFINITY, f3 = -INFINITY;
        for (int w = 0; w < kSW; ++w) {
            f0 = fminf(f0, L.pf[0][w]);
            f1 = fmaxf(f1, L.pf[1][w]);
            f2 = fminf(f2, L.pf[2][w]);
            f3 = fmaxf(f3, L.pf[3][w]);
        }
        st->SL = SL;
        st->SR = SR;
        st->nL = nL;
        st->nR = nR;
        st->nonfinite = nf;
        st->bmin = f0;
        st->bmax = f1;
        st->smin = f2;
        st->smax = f3;
    }
    // the tails as virtual end nodes (an infinite bracket end has none)
    Anch left = empty_pre(), right = empty_suf();
    bool hasL = false, hasR = false;
    if (a.tails) {
        if (nf) {
            if (tid == 0)
                st->solve_state = kSolveNonfinite;
            return false;
        }
        if (nB > (uint64_t)a.cap) {
            if (tid == 0)
                st->solve_state = kSolveOverflow;
            return false;
        }
        hasL = aL != -INFINITY;
        hasR = aR != INFINITY;
        if (hasL)
            left = node(aL, SL);
        if (hasR)
            right = node(aR, SR);
        if (a.direct) {
            // the whole band sorted and scanned at once
            if (nB > (uint64_t)kBucketCap) {
                if (tid == 0)
                    st->solve_state = kSolveDirectOverflow;
                return false;
            }
            job.xg = a.sorted;
            job.cntu = (int)nB;
            job.unsorted = true;
            job.certify = true;
            job.hasL = hasL;
            job.hasR = hasR;
            job.lo_node = left;
            job.Su = right;
            job.Cu = (uint32_t)nR;
            return true;
        }
    } else {
        nR = 0;
    }
    if (use_ref)
        return solve_level1_ref(a, L, job, mine, g0, ref, Eh, ref_scan_finish<kSW>(L.wt, rpart), left, right, nR);
    const Scan2 sc = scan2_finish<kSW>(L.wt, part1, c);
    const uint32_t NG = sc.cnt_all;
    const uint32_t cnt_before = sc.cnt_before;
    const Anch pre_before = fwd(left, sc.pre_before, c);  // everything before this thread's groups
    const Anch suf_after = bwd(sc.suf_after, right, c);   // everything after them

    // ---- bracket certificate (every thread, same values) ---------------------------
    if (a.tails) {
        const Anch Sall = bwd(sc.suf_all, right, c);
        const double mL = hasL ? mass_at(left.x, left.v, (double)NG + (double)nR, Sall, c) : (double)NG + (double)nR;
        const Anch Pall = fwd(left, sc.pre_all, c);
        double mR = 0.0;
        if (hasR)
            mR = (double)nR - 0.5 * right.v + 0.5 * Pall.v * exp2_nonpos(((double)Pall.x - (double)right.x) * c);
        if (tid == 0) {
            st->massL = mL;
            st->massR = mR;
        }
        const bool rejL = hasL && !(mL >= k);
        const bool rejR = !rejL && hasR && !(mR <= k);
        if (rejL || rejR) {
            if (tid == 0)
                st->solve_state = rejL ? kSolveRejectLow : kSolveRejectHigh;
            return false;
        }
    }

    // ---- masses at the group ends; the two groups around the root ----------------------
    int tc = -1, uc = T;
    if (gpt == 1) {
        if (g0 < T && mine.cnt) {
            const Anch P = fwd(pre_before, node(mine.hi, mine.TA), c);
            const uint32_t after = NG - (cnt_before + mine.cnt) + (uint32_t)nR;
            if (mass_at(mine.hi, P.v, (double)after, suf_after, c) >= k) {
                tc = g0;
                L.lo[tid] = P;
            } else {
                uc = g0;
                L.hi[tid].g = mine;
                L.hi[tid].Sx = suf_after.x;
                L.hi[tid].Sv = suf_after.v;
                L.hi[tid].Cafter = after;
            }
        }
    } else {
        // per-group suffixes through the scratch array, then the forward walk
        Anch cur = suf_after;
        for (int g = g1 - 1; g >= g0; --g) {
            const GroupAgg G = a.agg[g];
            a.scan[g].Sx = cur.x;
            a.scan[g].Sv = cur.v;
            if (G.cnt)
                cur = bwd(node(G.lo, G.TB), cur, c);
        }
        Anch P = pre_before;
        uint32_t through = cnt_before;
        for (int g = g0; g < g1; ++g) {
            const GroupAgg G = a.agg[g];
            if (!G.cnt)
                continue;
            through += G.cnt;
            const uint32_t after = NG - through + (uint32_t)nR;
            P = fwd(P, node(G.hi, G.TA), c);
            const Anch S = node((float)a.scan[g].Sx, a.scan[g].Sv);
            if (mass_at(G.hi, P.v, (double)after, S, c) >= k) {
                tc = g;
                L.lo[tid] = P;
            } else if (uc == T) {
                uc = g;
                L.hi[tid].g = G;
                L.hi[tid].Sx = S.x;
                L.hi[tid].Sv = S.v;
                L.hi[tid].Cafter = after;
            }
        }
    }
    int tstar, u;
    block_max_min(tc, uc, L, &tstar, &u);  // [1]
    if (u < tstar) {
        // rounding broke the monotone order of the group-end masses: take
        // the first non-empty group after t* instead
        __syncthreads();
        int mine_u = T;
        if (gpt == 1) {
            if (g0 < T && g0 > tstar && mine.cnt) {
                mine_u = g0;
                L.hi[tid].g = mine;
                L.hi[tid].Sx = suf_after.x;
                L.hi[tid].Sv = suf_after.v;
                L.hi[tid].Cafter = NG - (cnt_before + mine.cnt) + (uint32_t)nR;
            }
        } else {
            uint32_t through = cnt_before;
            for (int g = g0; g < g1; ++g) {
                const GroupAgg G = a.agg[g];
                through += G.cnt;
                if (g > tstar && G.cnt) {
                    mine_u = g;
                    L.hi[tid].g = G;
                    L.hi[tid].Sx = (float)a.scan[g].Sx;
                    L.hi[tid].Sv = a.scan[g].Sv;
                    L.hi[tid].Cafter = NG - through + (uint32_t)nR;
                    break;
                }
            }
        }
        int dummy;
        block_max_min(-1, mine_u, L, &dummy, &u);
    }
    Anch lo_node = left;
    if (tstar >= 0)
        lo_node = L.lo[tstar / gpt];
    if (u >= T) {
        // root between the last group and the right node
        if (tid == 0)
            finish(a, gap_root(lo_node, right, (double)nR, k, a.alpha, c));
        return false;
    }
    const RowHi Ur = L.hi[u / gpt];
    const GroupAgg U = Ur.g;
    const Anch Su = node(Ur.Sx, Ur.Sv);
    const uint32_t Cu = Ur.Cafter;
    if (U.lo == U.hi) {
        // every value of the group is equal: the root lies before it
        if (tid == 0)
            finish(a, gap_root(lo_node, bwd(node(U.lo, U.TB), Su, c), (double)U.cnt + (double)Cu, k, a.alpha, c));
        return false;
    }
    const int cntu = (int)U.cnt;
    if (cntu > kBucketCap) {
        if (tid == 0)
            st->solve_state = kSolveBucketOverflow;
        return false;
    }

    job.xg = a.sorted + U.start;
    job.cntu = cntu;
    job.unsorted = a.tails != 0;  // band buckets arrive unordered, full-sort tiles sorted
    job.certify = false;
    job.hasL = false;
    job.hasR = false;
    job.lo_node = lo_node;
    job.Su = Su;
    job.Cu = Cu;
    return true;
}

__global__ __launch_bounds__(kST) void solve_kernel(SolveArgs a)
{
    __shared__ SolveLds L;
    Level2Job job;
    if (solve_levels(a, L, job))
        level2(a, L, job);
    // every exit ends here: publish the status for the host
    __syncthreads();
    publish_status(a.st, a.mirror, a.seq);
}

hipError_t launch_solve(const SolveArgs& a, hipStream_t stream)
{
    STK_LAUNCH(kKSolve, stream, solve_kernel, dim3(1), dim3(kST), 0, stream, a);
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
