// rows.hip -- batched rows: many independent soft top-k problems at once.
//
// The aiqbench.com abstract and the gist.science summary of Fast LapSum
// (sections 1 and 2) name expert activation, token routing and attention
// pruning as the operator's workloads: many rows, each a small soft top-k
// with its own threshold.  Each row r of `rows` scores (row-major, n_row per
// row) gets b_r with sum_i F((s_ri - b_r)/alpha) = k, p_ri = F((s_ri -
// b_r)/alpha), and the VJP of each row as in the single-vector path.
//
// gfx950 design.  Three families of kernels, every one holding a row (or
// its share of one) in registers:
//   batched forward -- partition refinement, no sort (rows_refine_kernel:
//     lane groups of G lanes, several rows per wave, up to 2048 scores;
//     rows_refine_wg_kernel: one work-group per row beyond, in registers up
//     to 8192 scores and streamed after).  The row's split sums at a point
//     r give the closed-form root of the model that puts every score on its
//     side of r; the step repeats from that root until no score lies
//     between the point and its root, which is then the exact root.
//   sorted solve -- the one-kernel route of a single vector of at most
//     8192 scores (rows_group_forward_kernel up to 1024 scores,
//     rows_forward_kernel beyond): the row is loaded coalesced (R scores
//     per thread), copied as order-preserving keys and sorted by a bitonic
//     network in its direction-free form (the sorted keys end in blocked
//     order: thread t holds positions t*R .. t*R+R-1).  The full-sort solver
//     of section 2.2 then needs, at every breakpoint x_j, the left sum
//     A_j = sum_{i<=j} e^{(x_i-x_j)/alpha} and the right sum
//     sum_{i>j} e^{(x_j-x_i)/alpha}.  When the row spans at most kRowSpan
//     in log2 units ((x_max - x_min) log2(e)/alpha), every
//     E_i = e^{(x_i-x_r)/alpha} about the row's midpoint x_r and its
//     reciprocal are normal fp64 numbers, so both sums are plain prefix and
//     suffix sums of E and 1/E scaled by 1/E_j and E_j: one exponential per
//     score, fp64 additions in the scans.  Each E is an fp32 exp2 of the
//     fractional exponent times an exact power of two (relative error a few
//     fp32 ulps, which moves b by about 1e-7 alpha).  Wider rows take the
//     anchored sums of the single-vector segment solve (an exponential per
//     combination, any range).  The last breakpoint with mass >= k is found
//     by a block max and its owner applies the closed-form root (fp64).
//   backward -- each row's D and G, then its gradient (lane groups up to
//     1024 scores, one work-group per row up to 8192, a streamed work-group
//     beyond).
// p = F((s - b)/alpha) is emitted from the registers still holding the row
// in load order: s - b measured in fp64 (or from the fp32 split of b), the
// exponential in fp32.
#include <type_traits>

#include "stk_common.hpp"
#include "stk_layout.hpp"
#include "stk_prof.hpp"
#include "stk_scan.hpp"

namespace stk {

namespace {

// Largest row span, in log2 units, that the reference-point sums cover:
// about the midpoint every exponent lies in [-900, 900], so E and 1/E are
// normal fp64 numbers and row sums of them stay far from overflow.
constexpr double kRowSpan = 1800.0;

// p = F((s - b)/alpha): s - b in fp64, the exponential in fp32
__device__ __forceinline__ float row_p(float v, double b, double c)
{
    const double x = (double)v - b;
    const float e = __builtin_amdgcn_exp2f((float)(-fabs(x) * c));
    return x <= 0.0 ? 0.5f * e : 1.0f - 0.5f * e;
}

// E = 2^((x - xr) c) and 1/E: fp32 exp2 of the fractional exponent (in
// [-1/2, 1/2]) scaled by the exact power of two
__device__ __forceinline__ void ref_exp(float x, double xr, double c, double& e, double& ei)
{
    const double y = ((double)x - xr) * c;
    const double j = __builtin_rint(y);
    const float f = (float)(y - j);
    const int ij = (int)j;
    e = ldexp((double)__builtin_amdgcn_exp2f(f), ij);
    ei = ldexp((double)__builtin_amdgcn_exp2f(-f), -ij);
}

// Block scan of this thread's run sums: the sum of `ps` over earlier
// threads and of `ss` over later ones (exclusive both ways, additions only).
template <int kW>
__device__ __forceinline__ void scan_pair(double ps, double ss, double* wp, double* ws, double& pre, double& suf)
{
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    double p = ps, q = ss;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double op = __shfl_up(p, off, kWave);
        const double oq = __shfl_down(q, off, kWave);
        if (lane >= off)
            p += op;
        if (lane + off < kWave)
            q += oq;
    }
    double pe = __shfl_up(p, 1, kWave);
    double se = __shfl_down(q, 1, kWave);
    if (lane == 0)
        pe = 0.0;
    if (lane == kWave - 1)
        se = 0.0;
    if (kW > 1) {
        if (lane == kWave - 1)
            wp[wave] = p;
        if (lane == 0)
            ws[wave] = q;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kW; ++w) {
            if (w < wave)
                pe += wp[w];
            if (w > wave)
                se += ws[w];
        }
    }
    pre = pe;
    suf = se;
}

// d = e^{-|s-b|/alpha}/2 in fp32, s - b in fp64 (the single-vector VJP's)
__device__ __forceinline__ float row_d(float v, double b, double c)
{
    const float y = (float)(fabs((double)v - b) * c);
    return 0.5f * __builtin_amdgcn_exp2f(-y);
}

}  // namespace

// Ascending sort of a work-group's kT * R keys into blocked order (thread t
// ends with positions t * R .. t * R + R - 1): the bitonic network in its
// direction-free form (each merge compares the lower half with the mirror
// image of the upper half, then runs ascending half-cleaners).  Exchanges
// inside a thread are bare min/max, inside a wave lane shuffles, across
// waves one LDS round trip behind one barrier (two buffers used in turn).
// LDS holds element (t, r) at r * kT + t, so a wave touches distinct banks.
template <int kT, int R>
__device__ __forceinline__ void block_sort_flip(uint32_t (&v)[R], uint32_t* buf0, uint32_t* buf1)
{
    constexpr int N = kT * R;
    const int tid = threadIdx.x;
    int flip = 0;
#pragma unroll
    for (int k = 2; k <= N; k <<= 1) {
        if (k <= R) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int q = r ^ (k - 1);
                if ((r & (k >> 1)) == 0) {
                    const uint32_t lo = v[r] < v[q] ? v[r] : v[q];
                    const uint32_t hi = v[r] < v[q] ? v[q] : v[r];
                    v[r] = lo;
                    v[q] = hi;
                }
            }
        } else {
            // mirror partner: thread tid ^ (k / R - 1), register R - 1 - r
            const int d = k / R - 1;
            const bool lower = (tid & ((k >> 1) / R)) == 0;
            uint32_t o[R];
            if (d < kWave) {
#pragma unroll
                for (int r = 0; r < R; ++r)
                    o[r] = (uint32_t)__shfl_xor((int)v[R - 1 - r], d, kWave);
            } else {
                uint32_t* buf = flip ? buf1 : buf0;
                flip ^= 1;
#pragma unroll
                for (int r = 0; r < R; ++r)
                    buf[r * kT + tid] = v[r];
                __syncthreads();
#pragma unroll
                for (int r = 0; r < R; ++r)
                    o[r] = buf[(R - 1 - r) * kT + (tid ^ d)];
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
                v[r] = lower ? (v[r] < o[r] ? v[r] : o[r]) : (v[r] > o[r] ? v[r] : o[r]);
        }
#pragma unroll
        for (int j = k >> 2; j > 0; j >>= 1) {
            if (j < R) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if ((r & j) == 0) {
                        const uint32_t lo = v[r] < v[r | j] ? v[r] : v[r | j];
                        const uint32_t hi = v[r] < v[r | j] ? v[r | j] : v[r];
                        v[r] = lo;
                        v[r | j] = hi;
                    }
                }
            } else {
                const int d = j / R;
                const bool lower = (tid & d) == 0;
                uint32_t o[R];
                if (d < kWave) {
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        o[r] = (uint32_t)__shfl_xor((int)v[r], d, kWave);
                } else {
                    uint32_t* buf = flip ? buf1 : buf0;
                    flip ^= 1;
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        buf[r * kT + tid] = v[r];
                    __syncthreads();
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        o[r] = buf[r * kT + (tid ^ d)];
                }
#pragma unroll
                for (int r = 0; r < R; ++r)
                    v[r] = lower ? (v[r] < o[r] ? v[r] : o[r]) : (v[r] > o[r] ? v[r] : o[r]);
            }
        }
    }
}

// The root of one sorted row (blocked order, run e0 .. e0 + m - 1 in x) by
// reference-point sums; xs is the first point of the next run (if any).
template <int kT, int R>
__device__ __forceinline__ void solve_ref(const float (&x)[R], int e0, int m, float xs, float xmin, float xmax,
                                          const RowsArgs& a, double* wp, double* ws, int* imax, double* bsh)
{
    constexpr int kW = kT / kWave;
    const int n = a.n_row;
    const double c = a.log2e_over_alpha;
    const double xr = 0.5 * ((double)xmin + (double)xmax);
    // backward over the run: sv[r] = sum of 1/E after position r (kept), and
    // the run's sums of E and 1/E; E and 1/E are recomputed in the forward
    // pass below rather than kept (registers decide occupancy)
    double sv[R];
    double ps = 0.0, ss = 0.0;
#pragma unroll
    for (int r = R - 1; r >= 0; --r) {
        sv[r] = ss;
        if (r < m) {
            double e, ei;
            ref_exp(x[r], xr, c, e, ei);
            ps += e;
            ss += ei;
        }
    }
    double pre, suf;
    scan_pair<kW>(ps, ss, wp, ws, pre, suf);

    // mass at x_j: A_j / 2 + (points after j) - (right sum) / 2, with
    // A_j = P_{<=j} / E_j and right sum E_j S_{>j}; the gap's right end
    // carries S_{>j} E_{j+1}
    int jc = -1;
    Anch lo = empty_pre(), hi = empty_suf();
    double P = pre;
    double E0 = 0.0;
    double e, ei;
    ref_exp(x[0], xr, c, e, ei);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        double en = 0.0, ein = 0.0;
        if (r + 1 < R)
            ref_exp(x[r + 1], xr, c, en, ein);
        else if (e0 + R < n)
            ref_exp(xs, xr, c, en, ein);
        if (r == 0)
            E0 = e;
        if (r < m) {
            P += e;
            const double S = suf + sv[r];
            const double A = P * ei;
            if (0.5 * A + (double)(n - 1 - (e0 + r)) - 0.5 * (e * S) >= a.k) {
                jc = e0 + r;
                lo = node(x[r], A);
                hi = e0 + r + 1 < n ? node(r + 1 < R ? x[r + 1] : xs, S * en) : empty_suf();
            }
        }
        e = en;
        ei = ein;
    }
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    int jmax = jc;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const int o = __shfl_xor(jmax, off, kWave);
        jmax = o > jmax ? o : jmax;
    }
    if (kW > 1) {
        if (lane == 0)
            imax[wave] = jmax;
        __syncthreads();
        jmax = imax[0];
        for (int w = 1; w < kW; ++w)
            jmax = imax[w] > jmax ? imax[w] : jmax;
    }
    if (jmax >= 0) {
        if (jc == jmax)
            *bsh = gap_root(lo, hi, (double)(n - 1 - jmax), a.k, a.alpha, c);
    } else if (threadIdx.x == 0) {
        // the root lies before the first point: every point on the right
        *bsh = gap_root(empty_pre(), node(x[0], (suf + ss) * E0), (double)n, a.k, a.alpha, c);
    }
}

// The same root by anchored sums (any span): each combination rescales by
// an exponential of the anchor difference.
template <int kT, int R>
__device__ __forceinline__ void solve_anchored(const float (&x)[R], int e0, int m, const RowsArgs& a, WaveTot* wt,
                                               int* imax, double* bsh)
{
    constexpr int kW = kT / kWave;
    const int n = a.n_row;
    const double c = a.log2e_over_alpha;
    const double k = a.k;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    // backward chain within the run (suffix anchored at each element), then
    // the forward fold
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
    const Anch ex_suf = sc.suf_after;

    // breakpoint masses: the last one with mass >= k
    int jc = -1;
    Anch jlo = empty_pre(), jhi = empty_suf();
    Anch A = sc.pre_before;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r < m) {
            A = fwd(A, node(x[r], 1.0), c);
            const Anch Bn = r + 1 < m ? bwd(node(x[r + 1], bv[r + 1]), ex_suf, c) : ex_suf;
            if (mass_at(x[r], A.v, (double)(n - 1 - (e0 + r)), Bn, c) >= k) {
                jc = e0 + r;
                jlo = A;
                jhi = Bn;
            }
        }
    }
    int jmax = jc;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const int o = __shfl_xor(jmax, off, kWave);
        jmax = o > jmax ? o : jmax;
    }
    if (kW > 1) {
        if (lane == 0)
            imax[wave] = jmax;
        __syncthreads();
        jmax = imax[0];
        for (int w = 1; w < kW; ++w)
            jmax = imax[w] > jmax ? imax[w] : jmax;
    }
    if (jmax >= 0) {
        if (jc == jmax)
            *bsh = gap_root(jlo, jhi, (double)(n - 1 - jmax), k, a.alpha, c);
    } else if (threadIdx.x == 0) {
        // the root lies before the first point
        const Anch B0 = bwd(node(x[0], bv[0]), ex_suf, c);
        *bsh = gap_root(empty_pre(), B0, (double)n, k, a.alpha, c);
    }
}

// The single-vector route: the work-group's fp64 mass of p, then the
// status block (zeroed, then b, the mass, and the solve's outcome: a
// non-finite score shows as b = NaN) and its publication to the host.
template <int kT>
__device__ __forceinline__ void single_publish(const RowsArgs& a, double m, double b)
{
    constexpr int kW = kT / kWave;
    constexpr int kWords = (int)(sizeof(Status) / 4);
    __shared__ double red[kW];
    const int tid = threadIdx.x;
    m = wave_sum(m);
    if (lane_id() == 0)
        red[tid / kWave] = m;
    if (tid < kWords)
        reinterpret_cast<uint32_t*>(a.st)[tid] = 0u;
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
        for (int w = 0; w < kW; ++w)
            tot += red[w];
        const bool bad = b != b;
        a.st->b = b;
        a.st->mass = tot;
        a.st->emit_done = 1u;
        a.st->nonfinite = bad ? 1u : 0u;
        a.st->solve_state = bad ? kSolveNonfinite : kSolveOk;
    }
    __syncthreads();
    publish_status(a.st, a.mirror, a.seq);
}

template <int kT, int R>
__global__ __launch_bounds__(kT) void rows_forward_kernel(RowsArgs a)
{
    static_assert(kT * R <= kRowMax && (kT % kWave) == 0, "row shape");
    constexpr int kW = kT / kWave;
    __shared__ uint32_t buf0[kT * R];
    __shared__ uint32_t buf1[kT * R];
    __shared__ WaveTot wt[kW];
    __shared__ double wp[kW], ws[kW];
    __shared__ int imax[kW];
    __shared__ float first[kT];
    __shared__ float ends[2];
    __shared__ double bsh;
    const int tid = threadIdx.x;
    const int n = a.n_row;
    const double c = a.log2e_over_alpha;
    const int64_t row = blockIdx.x;
    const float* s = a.s + row * (int64_t)n;

    // the row in load order (coalesced), and as keys
    float vo[R];
    uint32_t key[R];
    bool bad = false;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = r * kT + tid;
        vo[r] = i < n ? s[i] : 0.0f;
        bad = bad || (i < n && !isfinite(vo[r]));
        key[r] = i < n ? float_to_key(vo[r]) : 0xFFFFFFFFu;
    }
    if (__syncthreads_or(bad)) {
        float* p = a.p + row * (int64_t)n;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = r * kT + tid;
            if (i < n)
                p[i] = NAN;
        }
        if (tid == 0)
            a.b[row] = NAN;
        if (a.st != nullptr)
            single_publish<kT>(a, 0.0, NAN);  // every thread is here: reports the non-finite score
        return;
    }
    block_sort_flip<kT, R>(key, buf0, buf1);

    // this thread's sorted run: positions e0 .. e0 + m - 1
    const int e0 = tid * R;
    const int m = n - e0 < 0 ? 0 : (n - e0 < R ? n - e0 : R);
    float x[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        x[r] = key_to_float(key[r]);
    // the row's ends and each run's first point
    first[tid] = x[0];
    if (tid == 0)
        ends[0] = x[0];
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (e0 + r == n - 1)
            ends[1] = x[r];
    __syncthreads();
    const float xmin = ends[0], xmax = ends[1];
    if (((double)xmax - (double)xmin) * c <= kRowSpan) {
        const float xs = e0 + R < n ? first[tid + 1] : INFINITY;
        solve_ref<kT, R>(x, e0, m, xs, xmin, xmax, a, wp, ws, imax, &bsh);
    } else {
        solve_anchored<kT, R>(x, e0, m, a, wt, imax, &bsh);
    }
    __syncthreads();
    const double b = bsh;
    if (tid == 0)
        a.b[row] = b;
    float* p = a.p + row * (int64_t)n;
    double mass = 0.0;  // this thread's share of the fp64 mass of p
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = r * kT + tid;
        if (i < n) {
            const float pv = row_p(vo[r], b, c);
            p[i] = pv;
            mass += (double)pv;
        }
    }
    if (a.st != nullptr)
        single_publish<kT>(a, mass, b);
}

// kVec: as in the lane-group backward, whole float4s per thread (thread t
// holds float4s u * kT + t) for rows of a multiple of 4 scores on aligned
// vectors.
template <int kT, int R, bool kVec>
__global__ __launch_bounds__(kT) void rows_backward_kernel(RowsArgs a)
{
    static_assert(!kVec || R % 4 == 0, "whole float4s per thread");
    constexpr int kW = kT / kWave;
    __shared__ double red[2][kW];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int n = a.n_row;
    const double c = a.log2e_over_alpha;
    const int64_t row = blockIdx.x;
    const float* s = a.s + row * (int64_t)n;
    const float* g = a.g + row * (int64_t)n;
    const double b = a.b_in[row];
    float dv[R], gv[R];
    double D = 0.0, G = 0.0;
    if (kVec) {
        const float4* s4 = reinterpret_cast<const float4*>(s);
        const float4* g4 = reinterpret_cast<const float4*>(g);
#pragma unroll
        for (int u = 0; u < R / 4; ++u) {
            const int q = u * kT + tid;
            const bool in = 4 * q < n;
            const float4 sq = in ? s4[q] : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 gq = in ? g4[q] : make_float4(0.f, 0.f, 0.f, 0.f);
            gv[4 * u + 0] = gq.x;
            gv[4 * u + 1] = gq.y;
            gv[4 * u + 2] = gq.z;
            gv[4 * u + 3] = gq.w;
            dv[4 * u + 0] = in ? row_d(sq.x, b, c) : 0.0f;
            dv[4 * u + 1] = in ? row_d(sq.y, b, c) : 0.0f;
            dv[4 * u + 2] = in ? row_d(sq.z, b, c) : 0.0f;
            dv[4 * u + 3] = in ? row_d(sq.w, b, c) : 0.0f;
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = r * kT + tid;
            const bool in = i < n;
            gv[r] = in ? g[i] : 0.0f;
            dv[r] = in ? row_d(s[i], b, c) : 0.0f;
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc_dg(dv[r], gv[r], D, G);
    D = wave_sum(D);
    G = wave_sum(G);
    if (lane == 0) {
        red[0][wave] = D;
        red[1][wave] = G;
    }
    __syncthreads();
    D = 0.0;
    G = 0.0;
    for (int w = 0; w < kW; ++w) {
        D += red[0][w];
        G += red[1][w];
    }
    const Ratio2 ratio = split_ratio(D > 0.0 ? G / D : 0.0);
    const float inv_alpha = (float)(1.0 / a.alpha);
    float* out = a.grad + row * (int64_t)n;
    if (kVec) {
        float4* o4 = reinterpret_cast<float4*>(out);
#pragma unroll
        for (int u = 0; u < R / 4; ++u) {
            const int q = u * kT + tid;
            if (4 * q < n)
                o4[q] = make_float4(dv[4 * u + 0] * inv_alpha * minus_ratio(gv[4 * u + 0], ratio),
                                    dv[4 * u + 1] * inv_alpha * minus_ratio(gv[4 * u + 1], ratio),
                                    dv[4 * u + 2] * inv_alpha * minus_ratio(gv[4 * u + 2], ratio),
                                    dv[4 * u + 3] * inv_alpha * minus_ratio(gv[4 * u + 3], ratio));
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = r * kT + tid;
            if (i < n)
                out[i] = dv[r] * inv_alpha * minus_ratio(gv[r], ratio);
        }
    }
}

// ---------------------------------------------------------------------------
// Rows of up to 1024 scores: G lanes per row (G a power of two up to 64),
// R scores per lane, 64 / G rows per wave.  Everything stays inside the
// lane group -- the sort's exchanges, the scans, the reductions -- so a
// wave needs no LDS and no barrier, and the work done once per row (the
// closed-form root, the scans' shuffle steps, the reductions) serves the
// wave's 64 / G rows in the same instructions.
// ---------------------------------------------------------------------------
constexpr int kGroupThreads = 256;

// lane mask of this lane's group
template <int G>
__device__ __forceinline__ uint64_t group_mask()
{
    if (G == kWave)
        return ~0ull;
    return ((1ull << G) - 1ull) << (lane_id() & ~(G - 1));
}

template <int G>
__device__ __forceinline__ bool group_any(bool v)
{
    return (__ballot(v) & group_mask<G>()) != 0ull;
}

template <int G>
__device__ __forceinline__ int group_max(int v)
{
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) {
        const int o = __shfl_xor(v, off, kWave);
        v = o > v ? o : v;
    }
    return v;
}

template <int G>
__device__ __forceinline__ double group_sum(double v)
{
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

// Ascending sort of the group's G * R keys (blocked order: group lane gl
// ends with positions gl * R .. gl * R + R - 1).  Bitonic network in its
// direction-free form: each merge of two sorted halves first compares every
// element of the lower half with its mirror image in the upper half, then
// runs ascending half-cleaners; every compare-exchange puts the minimum at
// the lower position.
template <int G, int R>
__device__ __forceinline__ void group_sort(uint32_t (&v)[R], int gl)
{
    constexpr int N = G * R;
#pragma unroll
    for (int k = 2; k <= N; k <<= 1) {
        if (k <= R) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int q = r ^ (k - 1);
                if ((r & (k >> 1)) == 0) {
                    const uint32_t lo = v[r] < v[q] ? v[r] : v[q];
                    const uint32_t hi = v[r] < v[q] ? v[q] : v[r];
                    v[r] = lo;
                    v[q] = hi;
                }
            }
        } else {
            // mirror partner: lane gl ^ (k / R - 1), register R - 1 - r
            const bool lower = (gl & ((k >> 1) / R)) == 0;
            uint32_t o[R];
#pragma unroll
            for (int r = 0; r < R; ++r)
                o[r] = (uint32_t)__shfl_xor((int)v[R - 1 - r], k / R - 1, kWave);
#pragma unroll
            for (int r = 0; r < R; ++r)
                v[r] = lower ? (v[r] < o[r] ? v[r] : o[r]) : (v[r] > o[r] ? v[r] : o[r]);
        }
#pragma unroll
        for (int j = k >> 2; j > 0; j >>= 1) {
            if (j < R) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if ((r & j) == 0) {
                        const uint32_t lo = v[r] < v[r | j] ? v[r] : v[r | j];
                        const uint32_t hi = v[r] < v[r | j] ? v[r | j] : v[r];
                        v[r] = lo;
                        v[r | j] = hi;
                    }
                }
            } else {
                const bool lower = (gl & (j / R)) == 0;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t o = (uint32_t)__shfl_xor((int)v[r], j / R, kWave);
                    v[r] = lower ? (v[r] < o ? v[r] : o) : (v[r] > o ? v[r] : o);
                }
            }
        }
    }
}

// The gap of the group's sorted row where the mass crosses k, by
// reference-point sums (span <= kRowSpan): on the lane that owns the gap's
// left end (group lane 0 when the root lies before the first point), lo and
// hi are the sums anchored at the gap's ends and C the points after it.
struct RowGap {
    Anch lo, hi;
    double C;
    int jstar;  // the gap's left end; -1: before the first point
};

template <int G, int R>
__device__ __forceinline__ RowGap group_gap_ref(const float (&x)[R], int gl, int e0, int m, float xs, float xmin,
                                                float xmax, int n, double k, double c)
{
    const double xr = 0.5 * ((double)xmin + (double)xmax);
    // backward over the run: sv[r] = sum of 1/E after position r (kept), and
    // the run's sums of E and 1/E; E and 1/E are recomputed in the forward
    // pass below rather than kept (registers decide occupancy here)
    double sv[R];
    double ps = 0.0, ss = 0.0;
#pragma unroll
    for (int r = R - 1; r >= 0; --r) {
        sv[r] = ss;
        if (r < m) {
            double e, ei;
            ref_exp(x[r], xr, c, e, ei);
            ps += e;
            ss += ei;
        }
    }
    // exclusive scans inside the group: E before this run, 1/E after it
    double p = ps, q = ss;
#pragma unroll
    for (int off = 1; off < G; off <<= 1) {
        const double op = __shfl_up(p, off, kWave);
        const double oq = __shfl_down(q, off, kWave);
        if (gl >= off)
            p += op;
        if (gl + off < G)
            q += oq;
    }
    double pre = __shfl_up(p, 1, kWave);
    double suf = __shfl_down(q, 1, kWave);
    if (gl == 0)
        pre = 0.0;
    if (gl == G - 1)
        suf = 0.0;

    // mass at x_j: A_j / 2 + (points after j) - (right sum) / 2, with
    // A_j = P_{<=j} / E_j and right sum E_j S_{>j}; the gap's right end
    // carries S_{>j} E_{j+1}
    int jc = -1;
    Anch lo = empty_pre(), hi = empty_suf();
    double P = pre;
    double E0 = 0.0;
    double e, ei;
    ref_exp(x[0], xr, c, e, ei);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        // E of the next point: this run's next, or the next run's first
        double en = 0.0, ein = 0.0;
        if (r + 1 < R)
            ref_exp(x[r + 1], xr, c, en, ein);
        else if (e0 + R < n)
            ref_exp(xs, xr, c, en, ein);
        if (r == 0)
            E0 = e;
        if (r < m) {
            P += e;
            const double S = suf + sv[r];
            const double A = P * ei;
            if (0.5 * A + (double)(n - 1 - (e0 + r)) - 0.5 * (e * S) >= k) {
                jc = e0 + r;
                lo = node(x[r], A);
                hi = e0 + r + 1 < n ? node(r + 1 < R ? x[r + 1] : xs, S * en) : empty_suf();
            }
        }
        e = en;
        ei = ein;
    }
    RowGap gp;
    gp.jstar = group_max<G>(jc);
    gp.lo = lo;
    gp.hi = hi;
    gp.C = (double)(n - 1 - gp.jstar);
    if (gp.jstar < 0) {
        gp.lo = empty_pre();
        gp.hi = node(x[0], (suf + ss) * E0);
        gp.C = (double)n;
    }
    return gp;
}

// The same gap by anchored sums (any span).
template <int G, int R>
__device__ __forceinline__ RowGap group_gap_anchored(const float (&x)[R], int gl, int e0, int m, int n, double k,
                                                     double c)
{
    const int lane = lane_id();
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
    Anch p = lp, q = ls;
#pragma unroll
    for (int off = 1; off < G; off <<= 1) {
        const Anch op = shfl_anch(p, gl >= off ? lane - off : lane);
        const Anch oq = shfl_anch(q, gl + off < G ? lane + off : lane);
        if (gl >= off)
            p = fwd(op, p, c);
        if (gl + off < G)
            q = bwd(q, oq, c);
    }
    Anch pre = shfl_anch(p, gl > 0 ? lane - 1 : lane);
    Anch suf = shfl_anch(q, gl < G - 1 ? lane + 1 : lane);
    if (gl == 0)
        pre = empty_pre();
    if (gl == G - 1)
        suf = empty_suf();

    int jc = -1;
    Anch jlo = empty_pre(), jhi = empty_suf();
    Anch A = pre;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r < m) {
            A = fwd(A, node(x[r], 1.0), c);
            const Anch Bn = r + 1 < m ? bwd(node(x[r + 1], bv[r + 1]), suf, c) : suf;
            if (mass_at(x[r], A.v, (double)(n - 1 - (e0 + r)), Bn, c) >= k) {
                jc = e0 + r;
                jlo = A;
                jhi = Bn;
            }
        }
    }
    RowGap gp;
    gp.jstar = group_max<G>(jc);
    gp.lo = jlo;
    gp.hi = jhi;
    gp.C = (double)(n - 1 - gp.jstar);
    if (gp.jstar < 0) {
        gp.lo = empty_pre();
        gp.hi = bwd(node(x[0], bv[0]), suf, c);
        gp.C = (double)n;
    }
    return gp;
}

// Four waves per SIMD: with 16 scores per lane the kernel needs about 166
// VGPRs (three waves); capping it at 128 costs a few spilled registers and
// measured 5-10% faster (the sort's shuffles and exponentials want the
// latency hiding of the fourth wave).
template <int G, int R>
__global__ __launch_bounds__(kGroupThreads) __attribute__((amdgpu_waves_per_eu(4))) void rows_group_forward_kernel(
    RowsArgs a)
{
    static_assert(G >= 1 && G <= kWave && (G & (G - 1)) == 0, "group size");
    const int lane = lane_id();
    const int gl = lane & (G - 1);
    const int base = lane & ~(G - 1);
    const int64_t row = (int64_t)blockIdx.x * (kGroupThreads / G) + threadIdx.x / G;
    const bool live = row < a.rows;
    const int n = a.n_row;
    const double c = a.log2e_over_alpha;
    const float* s = a.s + row * (int64_t)n;

    // the row in load order, and as keys
    float vo[R];
    uint32_t key[R];
    bool bad = false;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = r * G + gl;
        const bool in = live && i < n;
        vo[r] = in ? s[i] : 0.0f;
        bad = bad || (in && !isfinite(vo[r]));
        key[r] = in ? float_to_key(vo[r]) : 0xFFFFFFFFu;
    }
    bad = group_any<G>(bad);
    group_sort<G, R>(key, gl);

    const int e0 = gl * R;
    const int m = n - e0 < 0 ? 0 : (n - e0 < R ? n - e0 : R);
    float x[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        x[r] = key_to_float(key[r]);
    // the row's ends, and the first point of the next lane's run
    float xl = x[0];
#pragma unroll
    for (int r = 1; r < R; ++r)
        if (r == (n - 1) % R)
            xl = x[r];
    const float xmin = __shfl(x[0], base, kWave);
    const float xmax = __shfl(xl, base + (n - 1) / R, kWave);
    const float xs = __shfl(x[0], gl + 1 < G ? lane + 1 : lane, kWave);
    const RowGap gp = ((double)xmax - (double)xmin) * c <= kRowSpan
                          ? group_gap_ref<G, R>(x, gl, e0, m, xs, xmin, xmax, n, a.k, c)
                          : group_gap_anchored<G, R>(x, gl, e0, m, n, a.k, c);
    // every lane evaluates the closed form on its own (lo, hi); the owner's
    // is the root
    const double bl = gap_root(gp.lo, gp.hi, gp.C, a.k, a.alpha, c);
    double b = __shfl(bl, base + (gp.jstar >= 0 ? gp.jstar / R : 0), kWave);
    if (bad)
        b = NAN;
    if (!live)
        return;
    if (gl == 0)
        a.b[row] = b;
    float* p = a.p + row * (int64_t)n;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = r * G + gl;
        if (i < n)
            p[i] = bad ? NAN : row_p(vo[r], b, c);
    }
}

// kVec: rows of a multiple of 4 scores on 16-byte aligned vectors; each lane
// then moves whole float4s (lane gl holds float4s u * G + gl), which halves
// the memory instructions; the sums only change order.
template <int G, int R, bool kVec>
__global__ __launch_bounds__(kGroupThreads) void rows_group_backward_kernel(RowsArgs a)
{
    static_assert(!kVec || R % 4 == 0, "whole float4s per lane");
    const int gl = lane_id() & (G - 1);
    const int64_t row = (int64_t)blockIdx.x * (kGroupThreads / G) + threadIdx.x / G;
    const bool live = row < a.rows;
    const int n = a.n_row;
    const double c = a.log2e_over_alpha;
    const float* s = a.s + row * (int64_t)n;
    const float* g = a.g + row * (int64_t)n;
    const double b = live ? a.b_in[row] : 0.0;
    float dv[R], gv[R];
    if (kVec) {
        const float4* s4 = reinterpret_cast<const float4*>(s);
        const float4* g4 = reinterpret_cast<const float4*>(g);
#pragma unroll
        for (int u = 0; u < R / 4; ++u) {
            const int q = u * G + gl;
            const bool in = live && 4 * q < n;
            const float4 sq = in ? s4[q] : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 gq = in ? g4[q] : make_float4(0.f, 0.f, 0.f, 0.f);
            gv[4 * u + 0] = gq.x;
            gv[4 * u + 1] = gq.y;
            gv[4 * u + 2] = gq.z;
            gv[4 * u + 3] = gq.w;
            dv[4 * u + 0] = in ? row_d(sq.x, b, c) : 0.0f;
            dv[4 * u + 1] = in ? row_d(sq.y, b, c) : 0.0f;
            dv[4 * u + 2] = in ? row_d(sq.z, b, c) : 0.0f;
            dv[4 * u + 3] = in ? row_d(sq.w, b, c) : 0.0f;
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = r * G + gl;
            const bool in = live && i < n;
            gv[r] = in ? g[i] : 0.0f;
            dv[r] = in ? row_d(s[i], b, c) : 0.0f;
        }
    }
    double D = 0.0, Gs = 0.0;
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc_dg(dv[r], gv[r], D, Gs);
    D = group_sum<G>(D);
    Gs = group_sum<G>(Gs);
    if (!live)
        return;
    const Ratio2 ratio = split_ratio(D > 0.0 ? Gs / D : 0.0);
    const float inv_alpha = (float)(1.0 / a.alpha);
    float* out = a.grad + row * (int64_t)n;
    if (kVec) {
        float4* o4 = reinterpret_cast<float4*>(out);
#pragma unroll
        for (int u = 0; u < R / 4; ++u) {
            const int q = u * G + gl;
            if (4 * q < n)
                o4[q] = make_float4(dv[4 * u + 0] * inv_alpha * minus_ratio(gv[4 * u + 0], ratio),
                                    dv[4 * u + 1] * inv_alpha * minus_ratio(gv[4 * u + 1], ratio),
                                    dv[4 * u + 2] * inv_alpha * minus_ratio(gv[4 * u + 2], ratio),
                                    dv[4 * u + 3] * inv_alpha * minus_ratio(gv[4 * u + 3], ratio));
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = r * G + gl;
            if (i < n)
                out[i] = dv[r] * inv_alpha * minus_ratio(gv[r], ratio);
        }
    }
}

// ---------------------------------------------------------------------------
// Rows without a sort: partition refinement (the band's solve in
// partition_solve.hip) on each row, held by a lane group in registers.
// At a split point r the group sums A = sum over s > r of e^{-(s-r)/alpha}
// and B = sum over s <= r of e^{(s-r)/alpha}, counts N above r and finds
// the nearest scores on either side; the segment's closed form around r,
// N - (A/2) u + (B/2)/u = k with u = e^{(b-r)/alpha}, gives the next r; the
// pass whose root lies between those nearest scores has found b exactly.
// The steps move monotonically to b (each a one-sided bound), so they end.
// A pass costs one exponential per score and a few lane-group shuffles, not
// the sort network's ~log^2 n compare-exchanges.
//   terms -- each pass splits at an fp64 point r; the scores compare with
//     and are measured from the largest float rf <= r (the same split), a
//     lane's terms 2^{-|s - rf| log2(e)/alpha} in fp32 (the difference is
//     exact for s within a factor 2 of rf, else off by half an ulp; exp2 a
//     few ulps) summed over its R scores in fp32, the group's sums in fp64
//     and moved from rf to r by one exact-range factor.  Terms within a few
//     alpha of r carry relative errors of a few 1e-7, so b moves by about
//     1e-6 alpha at most (1e-5 alpha is the bar; the tests see 1e-7); a sum
//     that falls below 2^-100 takes the far-gap form below;
//   start -- each lane group solves a row, then the row one grid stride on
//     (rows are loaded, solved and emitted one at a time); the first row
//     starts at its maximum, each later one at the group's previous b
//     shifted by the change of the row mean (any start converges; a near
//     one in 2-4 passes);
//   far gaps -- when the sum a step rests on underflows about r (r lies in
//     a gap of tens of alpha or more), the next pass re-sums the same split
//     with each side measured from its nearest score and takes the
//     segment's closed form anchored at the gap's ends (gap_root, the
//     sorted kernels' form), which needs no sum about r.
// ---------------------------------------------------------------------------
namespace {

template <int G>
__device__ __forceinline__ float group_minf(float v)
{
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1)
        v = fminf(v, __shfl_xor(v, off, kWave));
    return v;
}

template <int G>
__device__ __forceinline__ float group_maxf(float v)
{
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

template <int G>
__device__ __forceinline__ float group_sumf(float v)
{
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

// The positive root u of (A/2) u^2 + d u - B/2 = 0 in its cancellation-free
// form, in fp32 (a few ulps).  With d = 0 (k a whole number equal to the
// count above the split) the discriminant is sqrt(A) sqrt(B): the product
// A B would leave the normal fp32 range when both sums are small (two scores
// tens of alpha from the split, b between them).  Any other d is at least
// an ulp of k, whose square dwarfs such a product.
__device__ __forceinline__ float row_root_u(float d, float A, float B)
{
    const float disc = d != 0.0f ? sqrtf(d * d + A * B) : sqrtf(A) * sqrtf(B);
    return d > 0.0f ? B / (d + disc) : (disc - d) / A;
}

// p = F((s - b)/alpha) for b = bf + sb alpha / log2(e), bf a float <= b and
// 0 <= sb small: (s - bf) in fp32 (exact for s within a factor 2 of bf),
// the exponential in fp32; to about 1e-7.
__device__ __forceinline__ float row_p_split(float v, float bf, float sb, float cf)
{
    const float x = (v - bf) * cf - sb;
    const float e = __builtin_amdgcn_exp2f(-fabsf(x));
    return v <= bf ? 0.5f * e : 1.0f - 0.5f * e;
}

template <int G>
__device__ __forceinline__ uint32_t group_sum_u32(uint32_t v)
{
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

constexpr float kRowIterTol = 0x1p-30f;  // convergence slack, in units of alpha
constexpr float kRowSumMin = 0x1p-100f;  // smallest sum taken as exact (normal, 2^26 above the fp32 minimum)
// Passes of model steps before a long row's split point bisects instead
// (the work-group form, rows over 2048 scores).  A model step crosses the
// scores between its split and the root only as far as their terms let it:
// with alpha far below the spacing of the scores it crosses about one per
// pass, so a start many scores away from b would take as many passes, each
// a sweep of the row.  Every step also bounds b from one side (the step moves
// toward b), so the row keeps a bracket of fp32 keys; bisecting it (from
// the finite floats, cut by the last step) isolates the gap that holds b in
// at most 33 more passes (each perhaps followed by a re-sum), where the
// closed form ends.
// A row of at most kRowMaxPasses - 8 scores ends within n + 8 model steps
// and does not bisect.
constexpr int kRowModelPasses = 8;
constexpr int kRowMaxPasses = kRowModelPasses + 2 * 34;

// The fp32 split point halfway, in key order, between two keys.
__device__ __forceinline__ double key_midpoint(uint32_t kl, uint32_t kh)
{
    return (double)key_to_float(kl + (kh - kl) / 2u);
}

}  // namespace

// The j-th largest of the group's values v (one per lane, descending
// bitonic network over the group's lanes), j in 1..G.
template <int G>
__device__ __forceinline__ float group_kth_largest(float v, int j)
{
    const int gl = lane_id() & (G - 1);
#pragma unroll
    for (int size = 2; size <= G; size <<= 1) {
#pragma unroll
        for (int stride = size / 2; stride > 0; stride >>= 1) {
            const float o = __shfl_xor(v, stride, kWave);
            const bool desc = (gl & size) == 0;  // this block sorts descending
            const bool low = (gl & stride) == 0;
            v = (low == desc) ? fmaxf(v, o) : fminf(v, o);
        }
    }
    return __shfl(v, (lane_id() & ~(G - 1)) + j - 1, kWave);
}

// kVec: rows of a multiple of 4 scores on 16-byte aligned vectors, moved as
// whole float4 (lane gl holds float4 u * G + gl); the refinement only needs
// the row as a set.
// kFull: n_row == G * R, every slot holds a score (no per-score guards).
template <int G, int R, bool kVec, bool kFull>
__global__ __launch_bounds__(kGroupThreads) __attribute__((amdgpu_waves_per_eu(R > 16 ? 3 : 4))) void
rows_refine_kernel(RowsArgs a)
{
    static_assert(G >= 1 && G <= kWave && (G & (G - 1)) == 0, "group size");
    static_assert(!kVec || R % 4 == 0, "whole float4s per lane");
    const int gl = lane_id() & (G - 1);
    const int n = kFull ? G * R : a.n_row;
    const double c = a.log2e_over_alpha;
    const double k = a.k;
    const double tol = (double)kRowIterTol * a.alpha;
    const float cf = (float)c;
    const int64_t stride = (int64_t)gridDim.x * (kGroupThreads / G);
    // each pass that does not end crosses a score (n <= 2048 here: a bounded
    // worst case; the work-group form bisects instead for longer rows)
    const int max_passes = n + 8;
    // rank, among the G lane maxima, that estimates b on a first row: a lane
    // holds a score above b with probability about 1 - e^{-k/G}
    const int jmax = (int)fmin((double)G, fmax(1.0, rint((double)G * (1.0 - exp(-k / (double)G)))));
    // which of the lane's R slots hold a score (the same for every row)
    bool in_[R];
#pragma unroll
    for (int q = 0; q < R; ++q)
        in_[q] = kFull || (kVec ? 4 * ((q / 4) * G + gl) < n : q * G + gl < n);
    auto load_row = [&](int64_t rw, float (&dst)[R]) {
        const float* s = a.s + rw * (int64_t)n;
        if (kVec) {
            const float4* s4 = reinterpret_cast<const float4*>(s);
#pragma unroll
            for (int u = 0; u < R / 4; ++u) {
                const float4 f = in_[4 * u] ? s4[u * G + gl] : make_float4(0.f, 0.f, 0.f, 0.f);
                dst[4 * u + 0] = f.x;
                dst[4 * u + 1] = f.y;
                dst[4 * u + 2] = f.z;
                dst[4 * u + 3] = f.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < R; ++q)
                dst[q] = in_[q] ? s[q * G + gl] : 0.0f;
        }
    };
    double b_prev = NAN, mean_prev = 0.0;
    int64_t row = (int64_t)blockIdx.x * (kGroupThreads / G) + threadIdx.x / G;
    float v[R];
    if (row < a.rows)
        load_row(row, v);
    for (; row < a.rows; row += stride) {
        // the next row's loads go out before this row's passes
        float nx[R];
        const bool more = row + stride < a.rows;
        if (more)
            load_row(row + stride, nx);
        bool bad = false;
        float vmax = -INFINITY, vsum = 0.0f;
#pragma unroll
        for (int q = 0; q < R; ++q) {
            bad = bad || (in_[q] && !isfinite(v[q]));
            vmax = in_[q] ? fmaxf(vmax, v[q]) : vmax;
            vsum += in_[q] ? v[q] : 0.0f;
        }
        bad = group_any<G>(bad);
        const double mean = group_sum<G>((double)vsum) / (double)n;
        double r;
        if (isfinite(b_prev)) {
            r = b_prev + (mean - mean_prev);
        } else if (k <= 4.0 * G) {
            r = (double)group_kth_largest<G>(vmax, jmax);
        } else {
            r = mean;
        }
        double b = NAN;
        // gap: this pass re-sums the last pass's split with each side
        // measured from its nearest score (glo, ghi) instead of from rf
        bool gap = false;
        float rf = 0.0f, glo = 0.0f, ghi = 0.0f;
        for (int pass = 0; pass < max_passes && !bad; ++pass) {
            // the split point r in fp64; the scores compare with and are
            // measured from rf, the largest float <= r (no float lies in
            // (rf, r], so the split is the same), and the sums are moved
            // from rf to r by 2^{+-(r - rf) c}.  Each lane's terms and sums
            // in fp32 (two partial sums each); the group's sums in fp32 to
            // steer, and in fp64 for the pass that ends.
            if (!gap)
                rf = __double2float_rd(r);
            const float ref_hi = gap ? ghi : rf, ref_lo = gap ? glo : rf;
            float Af[2] = {0.0f, 0.0f}, Bf[2] = {0.0f, 0.0f};
            uint32_t N = 0;
            float lo = -INFINITY, hi = INFINITY;
            // one pass's terms; kGap: each side measured from its nearest
            // score (a re-sum), else both from rf (the common case, one
            // select less per score)
            auto terms = [&](auto kGap) {
#pragma unroll
                for (int q = 0; q < R; ++q) {
                    if (in_[q]) {
                        const bool up = v[q] > rf;
                        const float ref = decltype(kGap)::value ? (up ? ref_hi : ref_lo) : rf;
                        const float e = __builtin_amdgcn_exp2f(-fabsf(v[q] - ref) * cf);
                        Af[q & 1] += up ? e : 0.0f;
                        Bf[q & 1] += up ? 0.0f : e;
                        N += up ? 1u : 0u;
                        // nearest scores by compare and select: fminf /
                        // fmaxf would first quieten both operands (two more
                        // instructions each); the scores are finite here
                        hi = up && v[q] < hi ? v[q] : hi;
                        lo = !up && v[q] > lo ? v[q] : lo;
                    }
                }
            };
            if (gap)
                terms(std::true_type{});
            else
                terms(std::false_type{});
            const float la = Af[0] + Af[1], lb = Bf[0] + Bf[1];
            N = group_sum_u32<G>(N);
            lo = group_maxf<G>(lo);
            hi = group_minf<G>(hi);
            double bn;
            if (gap) {
                // the segment's closed form with its sums anchored at the
                // gap's ends, as the sorted kernels take it
                bn = gap_root(node(lo, group_sum<G>((double)lb)), node(hi, group_sum<G>((double)la)), (double)N, k,
                              a.alpha, c);
                gap = false;
            } else {
                const float sh = (float)((r - (double)rf) * c);  // >= 0, below an ulp of r times c
                const float ga = group_sumf<G>(la) * __builtin_amdgcn_exp2f(sh);
                const float gb = group_sumf<G>(lb) * __builtin_amdgcn_exp2f(-sh);
                const float df = (float)(k - (double)N);
                float u = row_root_u(df, ga, gb);
                if (!(u > 0.0f && u < INFINITY && (df > 0.0f ? gb : ga) > kRowSumMin)) {
                    // the sum the root rests on underflowed (or lost its
                    // precision) about r: r lies in a gap of tens of alpha
                    // or more; the next pass re-sums this split from the
                    // gap's ends
                    gap = true;
                    glo = lo;
                    ghi = hi;
                    continue;
                }
                bn = r + a.alpha * (double)(__builtin_amdgcn_logf(u) * 0.6931471805599453f);
                if (bn >= (double)lo - tol && bn <= (double)hi + tol) {
                    // the end: the same root from fp64 group sums
                    const float fa = (float)group_sum<G>((double)la) * __builtin_amdgcn_exp2f(sh);
                    const float fb = (float)group_sum<G>((double)lb) * __builtin_amdgcn_exp2f(-sh);
                    u = row_root_u(df, fa, fb);
                    bn = r + a.alpha * (double)(__builtin_amdgcn_logf(u) * 0.6931471805599453f);
                }
            }
            if (bn >= (double)lo - tol && bn <= (double)hi + tol) {
                b = bn;
                break;
            }
            r = bn;
        }
        if (bad)
            b = NAN;
        if (gl == 0)
            a.b[row] = b;
        float* p = a.p + row * (int64_t)n;
        const float bf = isfinite(b) ? __double2float_rd(b) : (float)b;
        const float sb = isfinite(b) ? (float)((b - (double)bf) * c) : 0.0f;
        if (kVec) {
            float4* p4 = reinterpret_cast<float4*>(p);
#pragma unroll
            for (int u = 0; u < R / 4; ++u) {
                const int q4 = u * G + gl;
                if (kFull || 4 * q4 < n)
                    p4[q4] = bad ? make_float4(NAN, NAN, NAN, NAN)
                                 : make_float4(row_p_split(v[4 * u], bf, sb, cf), row_p_split(v[4 * u + 1], bf, sb, cf),
                                               row_p_split(v[4 * u + 2], bf, sb, cf),
                                               row_p_split(v[4 * u + 3], bf, sb, cf));
            }
        } else {
#pragma unroll
            for (int q = 0; q < R; ++q) {
                const int i = q * G + gl;
                if (kFull || i < n)
                    p[i] = bad ? NAN : row_p_split(v[q], bf, sb, cf);
            }
        }
        if (!bad && isfinite(b)) {
            b_prev = b;
            mean_prev = mean;
        }
        if (more) {
#pragma unroll
            for (int q = 0; q < R; ++q)
                v[q] = nx[q];
        }
    }
}

// ---------------------------------------------------------------------------
// Rows longer than a lane group holds: the same refinement with one
// work-group per row (kWgT threads; the work-group walks rows one grid
// stride apart).  Rows up to kWgT * R scores stay in registers; longer
// ones are streamed from memory on every pass (kStream), so any row length
// runs batched, with no host loop.  Reductions go through LDS (two
// barriers a pass).  A first row starts at the mean of the four waves'
// lane-maxima quantiles (k/4 of the row above b per wave), the mirrored
// lane-minima quantile when n - k is small, or the normal quantile of the
// row's mean and spread otherwise; later rows at the previous b shifted by
// the change of the row mean.
// ---------------------------------------------------------------------------
constexpr int kWgT = 256;

namespace {

struct WgRed {
    float f[4][kWgT / kWave];
    double d[2][kWgT / kWave];
    uint32_t u[kWgT / kWave];
};

// Work-group totals of one pass (every thread receives them): fp32 sums
// of the two sides, the count above, the nearest scores below and above.
__device__ __forceinline__ void wg_pass_totals(float& la, float& lb, uint32_t& N, float& lo, float& hi, WgRed& L)
{
    constexpr int kW = kWgT / kWave;
    const int wave = threadIdx.x / kWave;
    la = group_sumf<kWave>(la);
    lb = group_sumf<kWave>(lb);
    N = group_sum_u32<kWave>(N);
    lo = group_maxf<kWave>(lo);
    hi = group_minf<kWave>(hi);
    if (lane_id() == 0) {
        L.f[0][wave] = la;
        L.f[1][wave] = lb;
        L.f[2][wave] = lo;
        L.f[3][wave] = hi;
        L.u[wave] = N;
    }
    __syncthreads();
    la = lb = 0.0f;
    N = 0;
    lo = -INFINITY;
    hi = INFINITY;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
        la += L.f[0][w];
        lb += L.f[1][w];
        lo = fmaxf(lo, L.f[2][w]);
        hi = fminf(hi, L.f[3][w]);
        N += L.u[w];
    }
    __syncthreads();
}

// Work-group fp64 totals of two values.
__device__ __forceinline__ void wg_sum2(double& x, double& y, WgRed& L)
{
    constexpr int kW = kWgT / kWave;
    const int wave = threadIdx.x / kWave;
    x = group_sum<kWave>(x);
    y = group_sum<kWave>(y);
    if (lane_id() == 0) {
        L.d[0][wave] = x;
        L.d[1][wave] = y;
    }
    __syncthreads();
    x = y = 0.0;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
        x += L.d[0][w];
        y += L.d[1][w];
    }
    __syncthreads();
}

}  // namespace

template <int R, bool kStream>
__global__ __launch_bounds__(kWgT) void rows_refine_wg_kernel(RowsArgs a)
{
    __shared__ WgRed L;
    const int tid = threadIdx.x;
    const int n = a.n_row;
    const double c = a.log2e_over_alpha;
    const double k = a.k;
    const double tol = (double)kRowIterTol * a.alpha;
    const float cf = (float)c;
    const bool vec = (n % 4) == 0 && ((reinterpret_cast<uintptr_t>(a.s) | reinterpret_cast<uintptr_t>(a.p)) & 15u) == 0;
    // slot q of this thread: float4 q / 4 at (q / 4) * kWgT + tid, or the
    // single score q * kWgT + tid
    auto pos = [&](int q) -> int { return vec ? 4 * ((q / 4) * kWgT + tid) + (q & 3) : q * kWgT + tid; };
    // each model step that does not end crosses a score; past that bound,
    // bisection bounds the rest
    const bool may_bisect = n + 8 > kRowMaxPasses;
    const int max_passes = may_bisect ? kRowMaxPasses : n + 8;
    const double kw = k / (double)(kWgT / kWave);  // scores above b per wave's quarter
    const int jw = (int)fmin((double)kWave, fmax(1.0, rint((double)kWave * (1.0 - exp(-kw / (double)kWave)))));
    const double nkw = ((double)n - k) / (double)(kWgT / kWave);
    const int jwl = (int)fmin((double)kWave, fmax(1.0, rint((double)kWave * (1.0 - exp(-nkw / (double)kWave)))));
    double b_prev = NAN, mean_prev = 0.0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const float* s = a.s + row * (int64_t)n;
        float* p = a.p + row * (int64_t)n;
        float v[kStream ? 1 : R];
        // one sweep over this thread's scores: f(score) for each
        auto sweep = [&](auto&& f) {
            if (!kStream) {
#pragma unroll
                for (int q = 0; q < R; ++q)
                    if (pos(q) < n)
                        f(v[q]);
            } else if (vec) {
                const float4* s4 = reinterpret_cast<const float4*>(s);
                for (int i = tid; i < n / 4; i += kWgT) {
                    const float4 x = s4[i];
                    f(x.x);
                    f(x.y);
                    f(x.z);
                    f(x.w);
                }
            } else {
                for (int i = tid; i < n; i += kWgT)
                    f(s[i]);
            }
        };
        if (!kStream) {
            if (vec) {
                const float4* s4 = reinterpret_cast<const float4*>(s);
#pragma unroll
                for (int u = 0; u < R / 4; ++u) {
                    const int i4 = u * kWgT + tid;
                    const float4 x = 4 * i4 < n ? s4[i4] : make_float4(0.f, 0.f, 0.f, 0.f);
                    v[4 * u] = x.x;
                    v[4 * u + 1] = x.y;
                    v[4 * u + 2] = x.z;
                    v[4 * u + 3] = x.w;
                }
            } else {
#pragma unroll
                for (int q = 0; q < R; ++q)
                    v[q] = pos(q) < n ? s[pos(q)] : 0.0f;
            }
        }
        // the row's statistics: finiteness, mean and spread, each thread's
        // extremes
        float tmax = -INFINITY, tmin = INFINITY, tsum = 0.0f, tsq = 0.0f;
        bool tbad = false;
        sweep([&](float x) {
            tbad = tbad || !isfinite(x);
            tmax = fmaxf(tmax, x);
            tmin = fminf(tmin, x);
            tsum += x;
            tsq += x * x;
        });
        float est = 0.0f;
        if (kw <= 4.0 * kWave)
            est = group_kth_largest<kWave>(tmax, jw);
        else if (nkw <= 4.0 * kWave)
            est = -group_kth_largest<kWave>(-tmin, jwl);
        {
            double ds = tsum, dq = tsq;
            wg_sum2(ds, dq, L);
            tsum = (float)ds;
            tsq = (float)dq;
        }
        const double mean = (double)tsum / (double)n;
        {
            // the waves' estimates (one lane each) averaged; any bad score
            float e1 = lane_id() == 0 ? est : 0.0f, e2 = tbad ? 1.0f : 0.0f, e3 = 0.0f, e4 = 0.0f;
            uint32_t zu = 0;
            wg_pass_totals(e1, e2, zu, e3, e4, L);
            est = e1 / (float)(kWgT / kWave);
            tbad = e2 > 0.0f;
        }
        const bool bad = tbad;
        double r;
        if (isfinite(b_prev)) {
            r = b_prev + (mean - mean_prev);
        } else if (kw <= 4.0 * kWave || nkw <= 4.0 * kWave) {
            r = (double)est;
        } else {
            const double var = fmax((double)tsq / (double)n - mean * mean, 0.0);
            r = mean - sqrt(2.0 * var) * erfcinv(2.0 * (1.0 - k / (double)n));
        }
        double b = NAN;
        bool gap = false;
        float rf = 0.0f, glo = 0.0f, ghi = 0.0f;
        uint32_t kl = 0u, kh = 0xFFFFFFFFu;  // once bisecting: b lies in (key kl, key kh]
        bool bisect = false;
        for (int pass = 0; pass < max_passes && !bad; ++pass) {
            if (!gap)
                rf = __double2float_rd(r);
            const float ref_hi = gap ? ghi : rf, ref_lo = gap ? glo : rf;
            float Af = 0.0f, Bf = 0.0f;
            uint32_t N = 0;
            float lo = -INFINITY, hi = INFINITY;
            // kGap: each side measured from its nearest score (a re-sum),
            // else both from rf
            auto term = [&](float x, auto kGap) {
                const bool up = x > rf;
                const float ref = decltype(kGap)::value ? (up ? ref_hi : ref_lo) : rf;
                const float e = __builtin_amdgcn_exp2f(-fabsf(x - ref) * cf);
                Af += up ? e : 0.0f;
                Bf += up ? 0.0f : e;
                N += up ? 1u : 0u;
                hi = up && x < hi ? x : hi;  // compare and select (finite scores)
                lo = !up && x > lo ? x : lo;
            };
            if (gap)
                sweep([&](float x) { term(x, std::true_type{}); });
            else
                sweep([&](float x) { term(x, std::false_type{}); });
            const float la = Af, lb = Bf;
            float ga = la, gb = lb;
            wg_pass_totals(ga, gb, N, lo, hi, L);
            double bn;
            if (gap) {
                double A = la, B = lb;
                wg_sum2(A, B, L);
                bn = gap_root(node(lo, B), node(hi, A), (double)N, k, a.alpha, c);
                gap = false;
            } else {
                const float sh = (float)((r - (double)rf) * c);
                const float df = (float)(k - (double)N);
                float u = row_root_u(df, ga * __builtin_amdgcn_exp2f(sh), gb * __builtin_amdgcn_exp2f(-sh));
                if (!(u > 0.0f && u < INFINITY && (df > 0.0f ? gb : ga) > kRowSumMin)) {
                    gap = true;
                    glo = lo;
                    ghi = hi;
                    continue;
                }
                bn = r + a.alpha * (double)(__builtin_amdgcn_logf(u) * 0.6931471805599453f);
                if (bn >= (double)lo - tol && bn <= (double)hi + tol) {
                    double A = la, B = lb;
                    wg_sum2(A, B, L);
                    u = row_root_u(df, (float)A * __builtin_amdgcn_exp2f(sh), (float)B * __builtin_amdgcn_exp2f(-sh));
                    bn = r + a.alpha * (double)(__builtin_amdgcn_logf(u) * 0.6931471805599453f);
                }
            }
            if (bn >= (double)lo - tol && bn <= (double)hi + tol) {
                b = bn;
                break;
            }
            if (!may_bisect || pass + 1 < kRowModelPasses) {
                r = bn;
                continue;
            }
            if (!bisect) {
                // from here on the split bisects a bracket of b: the finite
                // floats, cut by the last model step (the steps all move one
                // way, toward b)
                kl = float_to_key(-0x1.fffffep127f);
                kh = float_to_key(0x1.fffffep127f);
                bisect = true;
            }
            // the step went toward b: b lies above r, or at most r
            if (bn > r)
                kl = max(kl, float_to_key(rf));
            else
                kh = min(kh, float_to_key(__double2float_ru(r)));
            r = kh > kl + 1u ? key_midpoint(kl, kh) : (double)key_to_float(kl);
        }
        if (bad)
            b = NAN;
        if (tid == 0)
            a.b[row] = b;
        const float bf = isfinite(b) ? __double2float_rd(b) : (float)b;
        const float sb = isfinite(b) ? (float)((b - (double)bf) * c) : 0.0f;
        if (!kStream) {
#pragma unroll
            for (int q = 0; q < R; ++q)
                if (pos(q) < n)
                    p[pos(q)] = bad ? NAN : row_p_split(v[q], bf, sb, cf);
        } else if (vec) {
            const float4* s4 = reinterpret_cast<const float4*>(s);
            float4* p4 = reinterpret_cast<float4*>(p);
            for (int i = tid; i < n / 4; i += kWgT) {
                const float4 x = s4[i];
                p4[i] = bad ? make_float4(NAN, NAN, NAN, NAN)
                            : make_float4(row_p_split(x.x, bf, sb, cf), row_p_split(x.y, bf, sb, cf),
                                          row_p_split(x.z, bf, sb, cf), row_p_split(x.w, bf, sb, cf));
            }
        } else {
            for (int i = tid; i < n; i += kWgT)
                p[i] = bad ? NAN : row_p_split(s[i], bf, sb, cf);
        }
        if (!bad && isfinite(b)) {
            b_prev = b;
            mean_prev = mean;
        }
    }
}

// The backward of rows longer than kRowMax: one work-group per row, the
// row streamed twice (D and G, then the gradient), the arithmetic of the
// other row backwards (fp32 d with s - b in fp64, fp64 sums with exact
// products, the ratio as a float pair).
__global__ __launch_bounds__(kWgT) void rows_backward_wg_kernel(RowsArgs a)
{
    __shared__ WgRed L;
    const int tid = threadIdx.x;
    const int n = a.n_row;
    const double c = a.log2e_over_alpha;
    const float inv_alpha = (float)(1.0 / a.alpha);
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const float* s = a.s + row * (int64_t)n;
        const float* g = a.g + row * (int64_t)n;
        float* out = a.grad + row * (int64_t)n;
        const double b = a.b_in[row];
        double D = 0.0, Gs = 0.0;
        for (int i = tid; i < n; i += kWgT)
            acc_dg(row_d(s[i], b, c), g[i], D, Gs);
        wg_sum2(D, Gs, L);
        const Ratio2 ratio = split_ratio(D > 0.0 ? Gs / D : 0.0);
        for (int i = tid; i < n; i += kWgT)
            out[i] = row_d(s[i], b, c) * inv_alpha * minus_ratio(g[i], ratio);
    }
}

namespace {

template <int kT, int R>
hipError_t launch_rows_t(const RowsArgs& a, bool forward, hipStream_t stream)
{
    constexpr bool kCanVec = R % 4 == 0;
    const bool vec = kCanVec && (a.n_row % 4) == 0 &&
                     ((reinterpret_cast<uintptr_t>(a.s) | reinterpret_cast<uintptr_t>(a.g) |
                       reinterpret_cast<uintptr_t>(a.grad)) & 15u) == 0;
    const dim3 grid((uint32_t)a.rows);
    if (forward)
        STK_LAUNCH(kKRowsForward, stream, (rows_forward_kernel<kT, R>), grid, dim3(kT), 0, stream, a);
    else if (vec)
        STK_LAUNCH(kKRowsBackward, stream, (rows_backward_kernel<kT, R, kCanVec>), grid, dim3(kT), 0, stream, a);
    else
        STK_LAUNCH(kKRowsBackward, stream, (rows_backward_kernel<kT, R, false>), grid, dim3(kT), 0, stream, a);
    return hipGetLastError();
}

template <int G, int R>
hipError_t launch_group_t(const RowsArgs& a, bool forward, hipStream_t stream)
{
    constexpr int kRows = kGroupThreads / G;
    const dim3 grid((uint32_t)((a.rows + kRows - 1) / kRows));
    const bool vec = (a.n_row % 4) == 0 &&
                     ((reinterpret_cast<uintptr_t>(a.s) | reinterpret_cast<uintptr_t>(a.g) |
                       reinterpret_cast<uintptr_t>(a.grad)) & 15u) == 0;
    if (forward)
        STK_LAUNCH(kKRowsForward, stream, (rows_group_forward_kernel<G, R>), grid, dim3(kGroupThreads), 0, stream, a);
    else if (vec)
        STK_LAUNCH(kKRowsBackward, stream, (rows_group_backward_kernel<G, R, true>), grid, dim3(kGroupThreads), 0,
                   stream, a);
    else
        STK_LAUNCH(kKRowsBackward, stream, (rows_group_backward_kernel<G, R, false>), grid, dim3(kGroupThreads), 0,
                   stream, a);
    return hipGetLastError();
}

// Forward shapes up to 1024 scores: 16 scores per lane from 33 on (the
// sort's in-register stages are its cheapest; fewer lanes per row share the
// per-row work among more rows), 4 or 8 below.
hipError_t launch_group_forward(const RowsArgs& a, hipStream_t stream)
{
    const int n = a.n_row;
    if (n <= 4)
        return launch_group_t<1, 4>(a, true, stream);
    if (n <= 8)
        return launch_group_t<2, 4>(a, true, stream);
    if (n <= 16)
        return launch_group_t<4, 4>(a, true, stream);
    if (n <= 32)
        return launch_group_t<4, 8>(a, true, stream);
    if (n <= 64)
        return launch_group_t<4, 16>(a, true, stream);
    if (n <= 128)
        return launch_group_t<8, 16>(a, true, stream);
    if (n <= 256)
        return launch_group_t<16, 16>(a, true, stream);
    if (n <= 512)
        return launch_group_t<32, 16>(a, true, stream);
    return launch_group_t<64, 16>(a, true, stream);
}

// Backward shapes up to 1024 scores: 4 scores per lane up to 256 (the
// widest lane groups read the row in the fewest, best-coalesced requests).
hipError_t launch_group_backward(const RowsArgs& a, hipStream_t stream)
{
    const int n = a.n_row;
    if (n <= 4)
        return launch_group_t<1, 4>(a, false, stream);
    if (n <= 8)
        return launch_group_t<2, 4>(a, false, stream);
    if (n <= 16)
        return launch_group_t<4, 4>(a, false, stream);
    if (n <= 32)
        return launch_group_t<8, 4>(a, false, stream);
    if (n <= 64)
        return launch_group_t<16, 4>(a, false, stream);
    if (n <= 128)
        return launch_group_t<32, 4>(a, false, stream);
    if (n <= 256)
        return launch_group_t<64, 4>(a, false, stream);
    if (n <= 512)
        return launch_group_t<64, 8>(a, false, stream);
    return launch_group_t<64, 16>(a, false, stream);
}

// The refinement forward: lane groups of G lanes, R scores each; the grid
// is what stays resident at once (four waves per SIMD at 16 scores per
// lane, three at 32), so each group walks several rows one grid stride
// apart and starts each at the last b.
template <int G, int R>
hipError_t launch_refine_t(const RowsArgs& a, hipStream_t stream)
{
    constexpr int kRows = kGroupThreads / G;
    const int64_t want = (a.rows + kRows - 1) / kRows;
    const int64_t cap = (int64_t)kCUs * (R > 16 ? 3 : 4);
    const dim3 grid((uint32_t)(want < cap ? want : cap));
    const bool vec = R % 4 == 0 && (a.n_row % 4) == 0 &&
                     ((reinterpret_cast<uintptr_t>(a.s) | reinterpret_cast<uintptr_t>(a.p)) & 15u) == 0;
    const bool full = a.n_row == G * R;
    if (vec && full)
        STK_LAUNCH(kKRowsForward, stream, (rows_refine_kernel<G, R, R % 4 == 0, true>), grid, dim3(kGroupThreads), 0,
                   stream, a);
    else if (vec)
        STK_LAUNCH(kKRowsForward, stream, (rows_refine_kernel<G, R, R % 4 == 0, false>), grid, dim3(kGroupThreads), 0,
                   stream, a);
    else
        STK_LAUNCH(kKRowsForward, stream, (rows_refine_kernel<G, R, false, false>), grid, dim3(kGroupThreads), 0,
                   stream, a);
    return hipGetLastError();
}

hipError_t launch_refine_forward(const RowsArgs& a, hipStream_t stream)
{
    const int n = a.n_row;
    if (n <= 4)
        return launch_refine_t<1, 4>(a, stream);
    if (n <= 8)
        return launch_refine_t<2, 4>(a, stream);
    if (n <= 16)
        return launch_refine_t<4, 4>(a, stream);
    if (n <= 32)
        return launch_refine_t<4, 8>(a, stream);
    if (n <= 64)
        return launch_refine_t<4, 16>(a, stream);
    if (n <= 128)
        return launch_refine_t<8, 16>(a, stream);
    if (n <= 256)
        return launch_refine_t<8, 32>(a, stream);
    if (n <= 512)
        return launch_refine_t<32, 16>(a, stream);
    if (n <= 1024)
        return launch_refine_t<64, 16>(a, stream);
    return launch_refine_t<64, 32>(a, stream);
}

}  // namespace

constexpr int kSingleThreads = 256;

__global__ __launch_bounds__(kSingleThreads) void single_status_kernel(SingleArgs a)
{
    constexpr int kW = kSingleThreads / kWave;
    constexpr int kWords = (int)(sizeof(Status) / 4);
    __shared__ double red[kW];
    const int tid = threadIdx.x;
    double m = 0.0;
    for (int64_t i = tid; i < a.n; i += kSingleThreads)
        m += (double)a.p[i];
    m = wave_sum(m);
    if (lane_id() == 0)
        red[tid / kWave] = m;
    if (tid < kWords)
        reinterpret_cast<uint32_t*>(a.st)[tid] = 0u;
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
        for (int w = 0; w < kW; ++w)
            tot += red[w];
        // the row kernel reports a non-finite score as b = NaN
        const double b = *a.b;
        const bool bad = b != b;
        a.st->b = b;
        a.st->mass = tot;
        a.st->emit_done = 1u;
        a.st->nonfinite = bad ? 1u : 0u;
        a.st->solve_state = bad ? kSolveNonfinite : kSolveOk;
    }
    __syncthreads();
    publish_status(a.st, a.mirror, a.seq);
}

// One row on its own (the single-vector route): the shortest chain per
// thread, up to 1024 threads with at most 4 scores each, then 512 threads
// with 16 (1024 threads with 8 would spill).
hipError_t launch_row_alone(const RowsArgs& a, bool forward, hipStream_t stream)
{
    const int n = a.n_row;
    if (n <= 64)
        return forward ? launch_group_forward(a, stream) : launch_group_backward(a, stream);
    if (n <= 256)
        return launch_rows_t<256, 1>(a, forward, stream);
    if (n <= 512)
        return launch_rows_t<512, 1>(a, forward, stream);
    if (n <= 1024)
        return launch_rows_t<1024, 1>(a, forward, stream);
    if (n <= 2048)
        return launch_rows_t<1024, 2>(a, forward, stream);
    if (n <= 4096)
        return launch_rows_t<1024, 4>(a, forward, stream);
    return launch_rows_t<512, 16>(a, forward, stream);
}

hipError_t launch_single_status(const SingleArgs& a, hipStream_t stream)
{
    single_status_kernel<<<1, kSingleThreads, 0, stream>>>(a);
    return hipGetLastError();
}

// The forward: rows up to 2048 scores refined in lane groups, longer rows
// by one work-group each (in registers up to 8192 scores, streamed beyond).
// The backward: lane groups up to 1024 scores, one work-group of 256
// threads (8 or 16 scores each) or 512 threads (16 each) per row up to
// kRowMax, and streamed work-groups beyond.
hipError_t launch_rows(const RowsArgs& a, bool forward, hipStream_t stream)
{
    const int n = a.n_row;
    if (forward && n <= kRefineRowMax)
        return launch_refine_forward(a, stream);
    if (forward) {
        // one work-group per row (resident work-groups walk the rows)
        const int64_t cap = (int64_t)kCUs * 4;
        const dim3 grid((uint32_t)(a.rows < cap ? a.rows : cap));
        if (n <= kWgT * 32)
            STK_LAUNCH(kKRowsForward, stream, (rows_refine_wg_kernel<32, false>), grid, dim3(kWgT), 0, stream, a);
        else
            STK_LAUNCH(kKRowsForward, stream, (rows_refine_wg_kernel<1, true>), grid, dim3(kWgT), 0, stream, a);
        return hipGetLastError();
    }
    if (n <= 1024)
        return launch_group_backward(a, stream);
    if (n <= 2048)
        return launch_rows_t<256, 8>(a, false, stream);
    if (n <= 4096)
        return launch_rows_t<256, 16>(a, false, stream);
    if (n <= kRowMax)
        return launch_rows_t<512, 16>(a, false, stream);
    const int64_t cap = (int64_t)kCUs * 4;
    STK_LAUNCH(kKRowsBackward, stream, rows_backward_wg_kernel, dim3((uint32_t)(a.rows < cap ? a.rows : cap)),
               dim3(kWgT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace stk
