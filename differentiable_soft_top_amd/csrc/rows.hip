// rows.hip -- batched rows: many independent soft top-k problems at once.
//
// The aiqbench.com abstract and the gist.science summary of Fast LapSum
// (sections 1 and 2) name expert activation, token routing and attention
// pruning as the operator's workloads: many rows, each a small soft top-k
// with its own threshold.  Each row r of `rows` scores (row-major, n_row per
// row) gets b_r with sum_i F((s_ri - b_r)/alpha) = k, p_ri = F((s_ri -
// b_r)/alpha), and the VJP of each row as in the single-vector path.
//
// gfx950 design: one work-group per row, the row held in registers.
//   forward -- the row is loaded coalesced (R scores per thread), copied as
//     order-preserving keys and sorted by a register bitonic network (the
//     sorted keys end in blocked order: thread t holds positions t*R ..
//     t*R+R-1).  Each thread folds its run forward and backward into
//     anchored sums; one work-group scan of those (the full-sort solver of
//     section 2.2: stable prefix/suffix sums of shifted exponentials) gives
//     every breakpoint's mass; the last breakpoint with mass >= k is found
//     by a block max and its owner applies the closed-form root (fp64).
//     p is then emitted from the registers still holding the row in load
//     order, in fp64 as in the single-vector emission.
//   backward -- d = e^{-|s-b|/alpha}/2 in fp32 (s - b in fp64), D and G
//     reduced in fp64 over the row, grad = (d/alpha)(g - G/D).
// No host synchronisation: a row holding a NaN or an infinite score gets
// b = NaN and p = NaN (the single-vector path reports ENONFINITE instead,
// which would need a read-back per call).
#include "stk_common.hpp"
#include "stk_layout.hpp"
#include "stk_prof.hpp"
#include "stk_scan.hpp"

namespace stk {

namespace {

// p = F((s - b)/alpha) in fp64 (the single-vector emission's arithmetic)
__device__ __forceinline__ float row_p(float v, double b, double c)
{
    const double x = (double)v - b;
    const double e = exp2_nonpos(-fabs(x) * c);
    return (float)(x <= 0.0 ? 0.5 * e : 1.0 - 0.5 * e);
}

// d = e^{-|s-b|/alpha}/2 in fp32, s - b in fp64 (the single-vector VJP's)
__device__ __forceinline__ float row_d(float v, double b, double c)
{
    const float y = (float)(fabs((double)v - b) * c);
    return 0.5f * __builtin_amdgcn_exp2f(-y);
}

}  // namespace

template <int kT, int R>
__global__ __launch_bounds__(kT) void rows_forward_kernel(RowsArgs a)
{
    static_assert(kT * R <= kRowMax && (kT % kWave) == 0, "row shape");
    constexpr int kW = kT / kWave;
    __shared__ uint32_t buf0[kT * R];
    __shared__ uint32_t buf1[kT * R];
    __shared__ WaveTot wt[kW];
    __shared__ int imax[kW];
    __shared__ double bsh;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int n = a.n_row;
    const double c = a.log2e_over_alpha;
    const double k = a.k;
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
        return;
    }
    block_bitonic_regs<kT, R>(key, buf0, buf1);

    // this thread's sorted run: positions e0 .. e0 + m - 1
    const int e0 = tid * R;
    const int m = n - e0 < 0 ? 0 : (n - e0 < R ? n - e0 : R);
    float x[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        x[r] = key_to_float(key[r]);
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
    // the block's last such breakpoint; its owner (whose own last one it
    // is) applies the closed form in the gap after it
    int jmax = jc;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const int o = __shfl_xor(jmax, off, kWave);
        jmax = o > jmax ? o : jmax;
    }
    if (lane == 0)
        imax[wave] = jmax;
    __syncthreads();
    int jstar = imax[0];
    for (int w = 1; w < kW; ++w)
        jstar = imax[w] > jstar ? imax[w] : jstar;
    if (jstar >= 0) {
        if (jc == jstar)
            bsh = gap_root(jlo, jhi, (double)(n - 1 - jstar), k, a.alpha, c);
    } else if (tid == 0) {
        // the root lies before the first point
        const Anch B0 = bwd(node(x[0], bv[0]), ex_suf, c);
        bsh = gap_root(empty_pre(), B0, (double)n, k, a.alpha, c);
    }
    __syncthreads();
    const double b = bsh;
    if (tid == 0)
        a.b[row] = b;
    float* p = a.p + row * (int64_t)n;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = r * kT + tid;
        if (i < n)
            p[i] = row_p(vo[r], b, c);
    }
}

template <int kT, int R>
__global__ __launch_bounds__(kT) void rows_backward_kernel(RowsArgs a)
{
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
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = r * kT + tid;
        const bool in = i < n;
        gv[r] = in ? g[i] : 0.0f;
        dv[r] = in ? row_d(s[i], b, c) : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        D += (double)dv[r];
        G += (double)(gv[r] * dv[r]);
    }
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
    const float ratio = D > 0.0 ? (float)(G / D) : 0.0f;
    const float inv_alpha = (float)(1.0 / a.alpha);
    float* out = a.grad + row * (int64_t)n;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = r * kT + tid;
        if (i < n)
            out[i] = dv[r] * inv_alpha * (gv[r] - ratio);
    }
}

namespace {

template <int kT, int R>
hipError_t launch_rows_t(const RowsArgs& a, bool forward, hipStream_t stream)
{
    if (forward)
        STK_LAUNCH(kKRowsForward, stream, (rows_forward_kernel<kT, R>), dim3((uint32_t)a.rows), dim3(kT), 0, stream, a);
    else
        STK_LAUNCH(kKRowsBackward, stream, (rows_backward_kernel<kT, R>), dim3((uint32_t)a.rows), dim3(kT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

// Work-group shape for a row: 64 threads up to 64 scores, 256 threads with
// up to 16 scores each up to 4096, 512 threads with 16 each up to 8192.
hipError_t launch_rows(const RowsArgs& a, bool forward, hipStream_t stream)
{
    const int n = a.n_row;
    if (n <= 64)
        return launch_rows_t<64, 1>(a, forward, stream);
    if (n <= 128)
        return launch_rows_t<64, 2>(a, forward, stream);
    if (n <= 256)
        return launch_rows_t<256, 1>(a, forward, stream);
    if (n <= 512)
        return launch_rows_t<256, 2>(a, forward, stream);
    if (n <= 1024)
        return launch_rows_t<256, 4>(a, forward, stream);
    if (n <= 2048)
        return launch_rows_t<256, 8>(a, forward, stream);
    if (n <= 4096)
        return launch_rows_t<256, 16>(a, forward, stream);
    return launch_rows_t<512, 16>(a, forward, stream);
}

}  // namespace stk
