// emit_vjp.hip -- the elementwise ends of the path.
//
// Emission (gist.science summary of Fast LapSum, section 2.1):
//     p_i = F((s_i - b)/alpha), F the standard Laplace CDF,
// with s_i - b taken in fp64 (b is fp64 and may sit within 1e-10 of an fp32
// score) and an fp64 exponential; the same pass sums p in fp64.  That sum is
// the certification pass of the aiqbench.com abstract: one more linear pass
// that checks the selected mass against k (here fused into emission, so it
// costs no extra read of s).
//
// Backward (section 2.1: the backward pass is analytic): implicit
// differentiation of sum_j F((s_j - b)/alpha) = k gives
//     grad_i = (d_i/alpha) (g_i - G/D),  d_i = e^{-|s_i - b|/alpha}/2,
//     D = sum d_i,  G = sum g_i d_i.
// Two streaming kernels: one reduces (D, G) in fp64 into per-work-group
// partials; the next has every work-group fold the partials in the same fixed
// order (so all agree bit for bit, with no ticket to initialise) and writes
// the gradient.  d_i only enters a 1e-4-relative result, so it uses the fp32
// hardware exponential.
#include "stk_common.hpp"
#include "stk_layout.hpp"
#include "stk_prof.hpp"

namespace stk {

// ---------------------------------------------------------------------------
__global__ void reset_status_kernel(Status* st, int open_bracket)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        if (open_bracket) {
            // a_L = a_R = +inf: pass-1 then folds every finite score into the
            // left tail (with zero weight) and only measures range/finiteness
            st->aL = INFINITY;
            st->aR = INFINITY;
        }
        st->nB = 0;
        st->solve_state = kSolveNotRun;
        st->emit_done = 0;
        st->ticket_radix = 0;
    }
}

hipError_t launch_reset_status(Status* st, hipStream_t stream, bool open_bracket)
{
    STK_LAUNCH(kKReset, stream, reset_status_kernel, dim3(1), dim3(64), 0, stream, st, open_bracket ? 1 : 0);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Streaming layout shared by the three kernels below: tiles of kB float4 per
// lane (kB * kStreamThreads float4 per work-group) taken in grid-stride
// order, so the resident work-groups sweep the vectors together.  Each tile's
// loads are all issued before its arithmetic, which then consumes them in
// arrival order; no load is left in flight across iterations (the compiler's
// wait counting would otherwise stall on it).  The ragged end (a partial tile
// and the last n mod 4 scores) goes, element by element, to the work-group
// whose next tile it would be.  Unaligned vectors take a plain element-wise
// grid-stride loop.  Large vectors use the larger batch.
//
// Direction: the emission re-reads the scores pass 1 has just streamed in
// ascending order, and the VJP's second pass re-reads the scores and the
// cotangent its first pass has just streamed in ascending order.  Both
// second passes walk their tiles in descending order, so they begin with the
// tiles most recently fetched, while those are still held in the caches
// (measured on MI355X at 10^8 scores: about 5 us off the emission and
// 15 us off the VJP's second pass).
namespace {

template <int kB>
__device__ __forceinline__ int64_t whole_tiles(int64_t n)
{
    return (n >> 2) / (kB * kStreamThreads);
}

// First element of the ragged end if this work-group owns it, else n.
template <int kB>
__device__ __forceinline__ int64_t ragged_start(int64_t n, int64_t T)
{
    const int64_t G = gridDim.x;
    return ((T - (int64_t)blockIdx.x) % G == 0) ? T * (kB * kStreamThreads) * 4 : n;
}

template <int kB>
__device__ __forceinline__ void load_q(const float4* __restrict__ p, int64_t t, float4 (&f)[kB])
{
#pragma unroll
    for (int u = 0; u < kB; ++u)
        f[u] = p[t * (kB * kStreamThreads) + u * kStreamThreads + threadIdx.x];
}

__device__ __forceinline__ float emit_one(float v, double b, double c, double& acc)
{
    const double x = (double)v - b;
    const double e = exp2_nonpos(-fabs(x) * c);  // e^{-|x|/alpha}
    const double p = x <= 0.0 ? 0.5 * e : 1.0 - 0.5 * e;
    acc += p;
    return (float)p;
}

// d = e^{-|s-b|/alpha}/2 in fp32 (s - b taken in fp64 first)
__device__ __forceinline__ float dens(float v, double b, double c)
{
    const float y = (float)(fabs((double)v - b) * c);
    return 0.5f * __builtin_amdgcn_exp2f(-y);
}

__device__ __forceinline__ void block_sum_to(double v, double* red, double* out)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    v = wave_sum(v);
    if (lane == 0)
        red[wave] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int w = 0; w < kStreamThreads / kWave; ++w)
            t += red[w];
        *out = t;
    }
}

}  // namespace

template <int kB, bool kVec, bool kNT>
__global__ __launch_bounds__(kStreamThreads) void emit_kernel(EmitArgs a)
{
    __shared__ double red[kStreamThreads / kWave];
    Status* st = a.st;
    if (st->solve_state != kSolveOk)
        return;
    const int tid = threadIdx.x;
    const double b = *a.b;
    const double c = a.log2e_over_alpha;
    const int64_t G = gridDim.x;
    double acc = 0.0;
    if (kVec) {
        const int64_t T = whole_tiles<kB>(a.n);
        const float4* s4 = reinterpret_cast<const float4*>(a.s);
        float4* p4 = reinterpret_cast<float4*>(a.p);
        for (int64_t t0 = blockIdx.x; t0 < T; t0 += G) {
            const int64_t t = T - 1 - t0;  // descending: see the note above
            float4 v[kB];
            load_q<kB>(s4, t, v);
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                float4 o;
                o.x = emit_one(v[u].x, b, c, acc);
                o.y = emit_one(v[u].y, b, c, acc);
                o.z = emit_one(v[u].z, b, c, acc);
                o.w = emit_one(v[u].w, b, c, acc);
                store4<kNT>(&p4[t * (kB * kStreamThreads) + u * kStreamThreads + tid], o);
            }
        }
        for (int64_t i = ragged_start<kB>(a.n, T) + tid; i < a.n; i += kStreamThreads)
            a.p[i] = emit_one(a.s[i], b, c, acc);
    } else {
        for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + tid; i < a.n; i += G * kStreamThreads)
            a.p[i] = emit_one(a.s[i], b, c, acc);
    }
    block_sum_to(acc, red, &a.partials[blockIdx.x]);
}

// Certification sum: one work-group folds the emission partials in fixed
// order into the status block.
__global__ __launch_bounds__(kStreamThreads) void emit_finalize_kernel(EmitArgs a)
{
    __shared__ double red[kStreamThreads / kWave];
    __shared__ double m;
    Status* st = a.st;
    if (st->solve_state != kSolveOk) {
        publish_status(st, a.mirror);
        return;
    }
    double t = 0.0;
    for (int i = threadIdx.x; i < a.blocks; i += kStreamThreads)
        t += a.partials[i];
    block_sum_to(t, red, &m);
    if (threadIdx.x == 0) {
        st->mass = m;
        st->emit_done = 1;
    }
    __syncthreads();
    publish_status(st, a.mirror);
}

hipError_t launch_emit(const EmitArgs& a, bool fold_mass, hipStream_t stream)
{
    const bool vec = ((reinterpret_cast<uintptr_t>(a.s) | reinterpret_cast<uintptr_t>(a.p)) & 15u) == 0;
    const dim3 grid(a.blocks), block(kStreamThreads);
    if (!vec)
        STK_LAUNCH(kKEmit, stream, (emit_kernel<1, false, false>), grid, block, 0, stream, a);
    else if (a.n >= kNontemporalMin)
        STK_LAUNCH(kKEmit, stream, (emit_kernel<kEmitBatchLarge, true, true>), grid, block, 0, stream, a);
    else if (a.n >= kStreamLargeMin)
        STK_LAUNCH(kKEmit, stream, (emit_kernel<kEmitBatchLarge, true, false>), grid, block, 0, stream, a);
    else
        STK_LAUNCH(kKEmit, stream, (emit_kernel<kEmitBatchSmall, true, false>), grid, block, 0, stream, a);
    if (fold_mass)
        STK_LAUNCH(kKEmitFinal, stream, emit_finalize_kernel, dim3(1), dim3(kStreamThreads), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
template <int kB, bool kVec>
__global__ __launch_bounds__(kStreamThreads) void vjp_reduce_kernel(VjpArgs a)
{
    __shared__ double red[2][kStreamThreads / kWave];
    const int tid = threadIdx.x;
    const double b = *a.b;
    const double c = a.log2e_over_alpha;
    const int64_t G = gridDim.x;
    double D = 0.0, G_ = 0.0;
    if (kVec) {
        const int64_t T = whole_tiles<kB>(a.n);
        const float4* s4 = reinterpret_cast<const float4*>(a.s);
        const float4* g4 = reinterpret_cast<const float4*>(a.g);
        for (int64_t t = blockIdx.x; t < T; t += G) {
            float4 vs[kB], vg[kB];
            load_q<kB>(s4, t, vs);
            load_q<kB>(g4, t, vg);
            // fp32 within a float4, fp64 across them
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                float d, dsum = 0.f, gsum = 0.f;
                d = dens(vs[u].x, b, c); dsum += d; gsum += vg[u].x * d;
                d = dens(vs[u].y, b, c); dsum += d; gsum += vg[u].y * d;
                d = dens(vs[u].z, b, c); dsum += d; gsum += vg[u].z * d;
                d = dens(vs[u].w, b, c); dsum += d; gsum += vg[u].w * d;
                D += (double)dsum;
                G_ += (double)gsum;
            }
        }
        for (int64_t i = ragged_start<kB>(a.n, T) + tid; i < a.n; i += kStreamThreads) {
            const float d = dens(a.s[i], b, c);
            D += (double)d;
            G_ += (double)(a.g[i] * d);
        }
    } else {
        for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + tid; i < a.n; i += G * kStreamThreads) {
            const float d = dens(a.s[i], b, c);
            D += (double)d;
            G_ += (double)(a.g[i] * d);
        }
    }
    block_sum_to(D, red[0], &a.partials[2 * blockIdx.x]);
    __syncthreads();
    block_sum_to(G_, red[1], &a.partials[2 * blockIdx.x + 1]);
}

template <int kB, bool kVec, bool kNT>
__global__ __launch_bounds__(kStreamThreads) void vjp_apply_kernel(VjpArgs a, int32_t reduce_blocks)
{
    __shared__ double red[2][kStreamThreads / kWave];
    __shared__ double tot[2];
    const int tid = threadIdx.x;
    // every work-group folds the partials in the same order
    double D = 0.0, G_ = 0.0;
    for (int i = tid; i < reduce_blocks; i += kStreamThreads) {
        D += a.partials[2 * i];
        G_ += a.partials[2 * i + 1];
    }
    block_sum_to(D, red[0], &tot[0]);
    __syncthreads();
    block_sum_to(G_, red[1], &tot[1]);
    __syncthreads();
    // every d_i underflowed (alpha tiny next to the gaps around b): the
    // gradient is then 0 everywhere and the ratio is irrelevant
    const float ratio = tot[0] > 0.0 ? (float)(tot[1] / tot[0]) : 0.0f;
    const float inv_alpha = (float)(1.0 / a.alpha);
    const double b = *a.b;
    const double c = a.log2e_over_alpha;
    const int64_t G = gridDim.x;
    if (kVec) {
        const int64_t T = whole_tiles<kB>(a.n);
        const float4* s4 = reinterpret_cast<const float4*>(a.s);
        const float4* g4 = reinterpret_cast<const float4*>(a.g);
        float4* o4 = reinterpret_cast<float4*>(a.grad);
        for (int64_t t0 = blockIdx.x; t0 < T; t0 += G) {
            const int64_t t = T - 1 - t0;  // descending: see the note above
            float4 vs[kB], vg[kB];
            load_q<kB>(s4, t, vs);
            load_q<kB>(g4, t, vg);
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                float4 o;
                o.x = dens(vs[u].x, b, c) * inv_alpha * (vg[u].x - ratio);
                o.y = dens(vs[u].y, b, c) * inv_alpha * (vg[u].y - ratio);
                o.z = dens(vs[u].z, b, c) * inv_alpha * (vg[u].z - ratio);
                o.w = dens(vs[u].w, b, c) * inv_alpha * (vg[u].w - ratio);
                store4<kNT>(&o4[t * (kB * kStreamThreads) + u * kStreamThreads + tid], o);
            }
        }
        for (int64_t i = ragged_start<kB>(a.n, T) + tid; i < a.n; i += kStreamThreads)
            a.grad[i] = dens(a.s[i], b, c) * inv_alpha * (a.g[i] - ratio);
    } else {
        for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + tid; i < a.n; i += G * kStreamThreads)
            a.grad[i] = dens(a.s[i], b, c) * inv_alpha * (a.g[i] - ratio);
    }
}

hipError_t launch_vjp(const VjpArgs& a, hipStream_t stream)
{
    const bool vec = ((reinterpret_cast<uintptr_t>(a.s) | reinterpret_cast<uintptr_t>(a.g) |
                       reinterpret_cast<uintptr_t>(a.grad)) & 15u) == 0;
    VjpArgs r = a;
    r.blocks = a.reduce_blocks;
    const dim3 block(kStreamThreads), gr(r.blocks), ga(a.blocks);
    if (!vec) {
        STK_LAUNCH(kKVjpReduce, stream, (vjp_reduce_kernel<1, false>), gr, block, 0, stream, r);
        STK_LAUNCH(kKVjpApply, stream, (vjp_apply_kernel<1, false, false>), ga, block, 0, stream, a, r.blocks);
    } else if (a.n >= kStreamLargeMin) {
        STK_LAUNCH(kKVjpReduce, stream, (vjp_reduce_kernel<kVjpBatchLarge, true>), gr, block, 0, stream, r);
        if (a.n >= kNontemporalMin)
            STK_LAUNCH(kKVjpApply, stream, (vjp_apply_kernel<kVjpBatchLarge, true, true>), ga, block, 0, stream, a,
                       r.blocks);
        else
            STK_LAUNCH(kKVjpApply, stream, (vjp_apply_kernel<kVjpBatchLarge, true, false>), ga, block, 0, stream, a,
                       r.blocks);
    } else {
        STK_LAUNCH(kKVjpReduce, stream, (vjp_reduce_kernel<kVjpBatchSmall, true>), gr, block, 0, stream, r);
        STK_LAUNCH(kKVjpApply, stream, (vjp_apply_kernel<kVjpBatchSmall, true, false>), ga, block, 0, stream, a,
                   r.blocks);
    }
    return hipGetLastError();
}

}  // namespace stk
