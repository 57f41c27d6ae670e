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
        st->ticket_pass1 = 0;
        st->ticket_hist = 0;
        st->ticket_emit = 0;
        st->ticket_radix = 0;
        st->ticket_tile = 0;
    }
}

hipError_t launch_reset_status(Status* st, hipStream_t stream, bool open_bracket)
{
    STK_LAUNCH(kKReset, stream, reset_status_kernel, dim3(1), dim3(64), 0, stream, st, open_bracket ? 1 : 0);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
namespace {

__device__ __forceinline__ float emit_one(float v, double b, double c, double& acc)
{
    const double x = (double)v - b;
    const double e = exp2_nonpos(-fabs(x) * c);  // e^{-|x|/alpha}
    const double p = x <= 0.0 ? 0.5 * e : 1.0 - 0.5 * e;
    acc += p;
    return (float)p;
}

}  // namespace

template <bool kVec, bool kNT>
__global__ __launch_bounds__(kStreamThreads) void emit_kernel(EmitArgs a)
{
    __shared__ double red[kStreamThreads / kWave];
    Status* st = a.st;
    if (st->solve_state != kSolveOk)
        return;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const double b = *a.b;
    const double c = a.log2e_over_alpha;
    double acc = 0.0;

    const int64_t n4 = a.n >> 2;
    const int64_t q0 = (n4 * blockIdx.x) / a.blocks;
    const int64_t q1 = (n4 * (blockIdx.x + 1)) / a.blocks;
    const float4* s4 = reinterpret_cast<const float4*>(a.s);
    float4* p4 = reinterpret_cast<float4*>(a.p);
    int64_t q = q0 + tid;
    for (; q + 3 * kStreamThreads < q1; q += 4 * kStreamThreads) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (kVec) {
                v[u] = s4[q + u * kStreamThreads];
            } else {
                const float* s = a.s + 4 * (q + u * kStreamThreads);
                v[u] = make_float4(s[0], s[1], s[2], s[3]);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float4 o;
            o.x = emit_one(v[u].x, b, c, acc);
            o.y = emit_one(v[u].y, b, c, acc);
            o.z = emit_one(v[u].z, b, c, acc);
            o.w = emit_one(v[u].w, b, c, acc);
            if (kVec) {
                store4<kNT>(&p4[q + u * kStreamThreads], o);
            } else {
                float* p = a.p + 4 * (q + u * kStreamThreads);
                p[0] = o.x;
                p[1] = o.y;
                p[2] = o.z;
                p[3] = o.w;
            }
        }
    }
    for (; q < q1; q += kStreamThreads) {
        float4 v;
        if (kVec) {
            v = s4[q];
        } else {
            const float* s = a.s + 4 * q;
            v = make_float4(s[0], s[1], s[2], s[3]);
        }
        float4 o;
        o.x = emit_one(v.x, b, c, acc);
        o.y = emit_one(v.y, b, c, acc);
        o.z = emit_one(v.z, b, c, acc);
        o.w = emit_one(v.w, b, c, acc);
        if (kVec) {
            store4<kNT>(&p4[q], o);
        } else {
            float* p = a.p + 4 * q;
            p[0] = o.x;
            p[1] = o.y;
            p[2] = o.z;
            p[3] = o.w;
        }
    }
    if (blockIdx.x == a.blocks - 1 && tid < 4) {
        const int64_t i = 4 * n4 + tid;
        if (i < a.n)
            a.p[i] = emit_one(a.s[i], b, c, acc);
    }

    acc = wave_sum(acc);
    if (lane == 0)
        red[wave] = acc;
    __syncthreads();
    if (tid == 0) {
        double t = 0.0;
        for (int w = 0; w < kStreamThreads / kWave; ++w)
            t += red[w];
        a.partials[blockIdx.x] = t;
    }
}

// Certification sum: one work-group folds the emission partials in fixed
// order into the status block.
__global__ __launch_bounds__(kStreamThreads) void emit_finalize_kernel(EmitArgs a)
{
    __shared__ double red[kStreamThreads / kWave];
    Status* st = a.st;
    if (st->solve_state != kSolveOk)
        return;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    double t = 0.0;
    for (int i = tid; i < a.blocks; i += kStreamThreads)
        t += a.partials[i];
    t = wave_sum(t);
    if (lane == 0)
        red[wave] = t;
    __syncthreads();
    if (tid == 0) {
        double m = 0.0;
        for (int w = 0; w < kStreamThreads / kWave; ++w)
            m += red[w];
        st->mass = m;
        st->emit_done = 1;
    }
}

hipError_t launch_emit(const EmitArgs& a, hipStream_t stream)
{
    const bool vec = ((reinterpret_cast<uintptr_t>(a.s) | reinterpret_cast<uintptr_t>(a.p)) & 15u) == 0;
    const bool nt = a.n >= kNontemporalMin;
    if (vec && nt)
        STK_LAUNCH(kKEmit, stream, (emit_kernel<true, true>), dim3(a.blocks), dim3(kStreamThreads), 0, stream, a);
    else if (vec)
        STK_LAUNCH(kKEmit, stream, (emit_kernel<true, false>), dim3(a.blocks), dim3(kStreamThreads), 0, stream, a);
    else
        STK_LAUNCH(kKEmit, stream, (emit_kernel<false, false>), dim3(a.blocks), dim3(kStreamThreads), 0, stream, a);
    STK_LAUNCH(kKEmitFinal, stream, emit_finalize_kernel, dim3(1), dim3(kStreamThreads), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
namespace {

// d = e^{-|s-b|/alpha}/2 in fp32 (s - b taken in fp64 first)
__device__ __forceinline__ float dens(float v, double b, double c)
{
    const float y = (float)(fabs((double)v - b) * c);
    return 0.5f * __builtin_amdgcn_exp2f(-y);
}

}  // namespace

template <bool kVec>
__global__ __launch_bounds__(kStreamThreads) void vjp_reduce_kernel(VjpArgs a)
{
    __shared__ double red[2][kStreamThreads / kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const double b = *a.b;
    const double c = a.log2e_over_alpha;
    double D = 0.0, G = 0.0;
    const int64_t n4 = a.n >> 2;
    const int64_t q0 = (n4 * blockIdx.x) / a.blocks;
    const int64_t q1 = (n4 * (blockIdx.x + 1)) / a.blocks;
    const float4* s4 = reinterpret_cast<const float4*>(a.s);
    const float4* g4 = reinterpret_cast<const float4*>(a.g);
    int64_t q = q0 + tid;
    for (; q + kStreamThreads < q1; q += 2 * kStreamThreads) {
        float4 v0, v1, w0, w1;
        if (kVec) {
            v0 = s4[q];
            v1 = s4[q + kStreamThreads];
            w0 = g4[q];
            w1 = g4[q + kStreamThreads];
        } else {
            const float* s = a.s + 4 * q;
            const float* g = a.g + 4 * q;
            v0 = make_float4(s[0], s[1], s[2], s[3]);
            w0 = make_float4(g[0], g[1], g[2], g[3]);
            s += 4 * kStreamThreads;
            g += 4 * kStreamThreads;
            v1 = make_float4(s[0], s[1], s[2], s[3]);
            w1 = make_float4(g[0], g[1], g[2], g[3]);
        }
        float d;
        float dsum = 0.f, gsum = 0.f;
        d = dens(v0.x, b, c); dsum += d; gsum += w0.x * d;
        d = dens(v0.y, b, c); dsum += d; gsum += w0.y * d;
        d = dens(v0.z, b, c); dsum += d; gsum += w0.z * d;
        d = dens(v0.w, b, c); dsum += d; gsum += w0.w * d;
        d = dens(v1.x, b, c); dsum += d; gsum += w1.x * d;
        d = dens(v1.y, b, c); dsum += d; gsum += w1.y * d;
        d = dens(v1.z, b, c); dsum += d; gsum += w1.z * d;
        d = dens(v1.w, b, c); dsum += d; gsum += w1.w * d;
        D += (double)dsum;
        G += (double)gsum;
    }
    for (; q < q1; q += kStreamThreads) {
        float4 v, w;
        if (kVec) {
            v = s4[q];
            w = g4[q];
        } else {
            const float* s = a.s + 4 * q;
            const float* g = a.g + 4 * q;
            v = make_float4(s[0], s[1], s[2], s[3]);
            w = make_float4(g[0], g[1], g[2], g[3]);
        }
        float d;
        float dsum = 0.f, gsum = 0.f;
        d = dens(v.x, b, c); dsum += d; gsum += w.x * d;
        d = dens(v.y, b, c); dsum += d; gsum += w.y * d;
        d = dens(v.z, b, c); dsum += d; gsum += w.z * d;
        d = dens(v.w, b, c); dsum += d; gsum += w.w * d;
        D += (double)dsum;
        G += (double)gsum;
    }
    if (blockIdx.x == a.blocks - 1 && tid < 4) {
        const int64_t i = 4 * n4 + tid;
        if (i < a.n) {
            const float d = dens(a.s[i], b, c);
            D += (double)d;
            G += (double)(a.g[i] * d);
        }
    }
    D = wave_sum(D);
    G = wave_sum(G);
    if (lane == 0) {
        red[0][wave] = D;
        red[1][wave] = G;
    }
    __syncthreads();
    if (tid == 0) {
        double td = 0.0, tg = 0.0;
        for (int w = 0; w < kStreamThreads / kWave; ++w) {
            td += red[0][w];
            tg += red[1][w];
        }
        a.partials[2 * blockIdx.x] = td;
        a.partials[2 * blockIdx.x + 1] = tg;
    }
}

template <bool kVec, bool kNT>
__global__ __launch_bounds__(kStreamThreads) void vjp_apply_kernel(VjpArgs a, int32_t reduce_blocks)
{
    __shared__ double red[2][kStreamThreads / kWave];
    __shared__ float coef[2];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    // every work-group folds the partials in the same order
    double D = 0.0, G = 0.0;
    for (int i = tid; i < reduce_blocks; i += kStreamThreads) {
        D += a.partials[2 * i];
        G += a.partials[2 * i + 1];
    }
    D = wave_sum(D);
    G = wave_sum(G);
    if (lane == 0) {
        red[0][wave] = D;
        red[1][wave] = G;
    }
    __syncthreads();
    if (tid == 0) {
        double td = 0.0, tg = 0.0;
        for (int w = 0; w < kStreamThreads / kWave; ++w) {
            td += red[0][w];
            tg += red[1][w];
        }
        // every d_i underflowed (alpha tiny next to the gaps around b): the
        // gradient is then 0 everywhere and the ratio is irrelevant
        coef[0] = td > 0.0 ? (float)(tg / td) : 0.0f;
        coef[1] = (float)(1.0 / a.alpha);
    }
    __syncthreads();
    const float ratio = coef[0];
    const float inv_alpha = coef[1];
    const double b = *a.b;
    const double c = a.log2e_over_alpha;

    const int64_t n4 = a.n >> 2;
    const int64_t q0 = (n4 * blockIdx.x) / a.blocks;
    const int64_t q1 = (n4 * (blockIdx.x + 1)) / a.blocks;
    const float4* s4 = reinterpret_cast<const float4*>(a.s);
    const float4* g4 = reinterpret_cast<const float4*>(a.g);
    float4* o4 = reinterpret_cast<float4*>(a.grad);
    for (int64_t q = q0 + tid; q < q1; q += kStreamThreads) {
        float4 v, w;
        if (kVec) {
            v = s4[q];
            w = g4[q];
        } else {
            const float* s = a.s + 4 * q;
            const float* g = a.g + 4 * q;
            v = make_float4(s[0], s[1], s[2], s[3]);
            w = make_float4(g[0], g[1], g[2], g[3]);
        }
        float4 o;
        o.x = dens(v.x, b, c) * inv_alpha * (w.x - ratio);
        o.y = dens(v.y, b, c) * inv_alpha * (w.y - ratio);
        o.z = dens(v.z, b, c) * inv_alpha * (w.z - ratio);
        o.w = dens(v.w, b, c) * inv_alpha * (w.w - ratio);
        if (kVec) {
            store4<kNT>(&o4[q], o);
        } else {
            float* p = a.grad + 4 * q;
            p[0] = o.x;
            p[1] = o.y;
            p[2] = o.z;
            p[3] = o.w;
        }
    }
    if (blockIdx.x == a.blocks - 1 && tid < 4) {
        const int64_t i = 4 * n4 + tid;
        if (i < a.n)
            a.grad[i] = dens(a.s[i], b, c) * inv_alpha * (a.g[i] - ratio);
    }
}

hipError_t launch_vjp(const VjpArgs& a, hipStream_t stream)
{
    const bool vec = ((reinterpret_cast<uintptr_t>(a.s) | reinterpret_cast<uintptr_t>(a.g) |
                       reinterpret_cast<uintptr_t>(a.grad)) & 15u) == 0;
    VjpArgs r = a;
    r.blocks = a.reduce_blocks;
    if (vec) {
        STK_LAUNCH(kKVjpReduce, stream, vjp_reduce_kernel<true>, dim3(r.blocks), dim3(kStreamThreads), 0, stream, r);
        if (a.n >= kNontemporalMin)
            STK_LAUNCH(kKVjpApply, stream, (vjp_apply_kernel<true, true>), dim3(a.blocks), dim3(kStreamThreads), 0,
                       stream, a, r.blocks);
        else
            STK_LAUNCH(kKVjpApply, stream, (vjp_apply_kernel<true, false>), dim3(a.blocks), dim3(kStreamThreads), 0,
                       stream, a, r.blocks);
    } else {
        STK_LAUNCH(kKVjpReduce, stream, vjp_reduce_kernel<false>, dim3(r.blocks), dim3(kStreamThreads), 0, stream, r);
        STK_LAUNCH(kKVjpApply, stream, (vjp_apply_kernel<false, false>), dim3(a.blocks), dim3(kStreamThreads), 0,
                   stream, a, r.blocks);
    }
    return hipGetLastError();
}

}  // namespace stk
