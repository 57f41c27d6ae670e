// stk_reduce.hpp -- fixed-order fold of the pass-1 per-work-group partials.
#pragma once

#include "stk_common.hpp"
#include "stk_layout.hpp"

namespace stk {

// One work-group folds the pass-1 partials in fixed order (each thread a
// strided subset, then fixed butterflies) and writes the totals to the
// status block.  Every thread returns the totals.
__device__ inline Pass1Partial reduce_pass1(const Pass1Partial* __restrict__ partials, int blocks, Status* st)
{
    constexpr int kMaxWaves = 16;
    __shared__ double rd[2][kMaxWaves];
    __shared__ unsigned long long rl[2][kMaxWaves];
    __shared__ uint32_t ru[kMaxWaves];
    __shared__ float rf[4][kMaxWaves];
    __shared__ Pass1Partial out;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int nw = blockDim.x / kWave;
    double SL = 0.0, SR = 0.0;
    unsigned long long nL = 0, nR = 0;
    uint32_t nf = 0;
    float bmin = INFINITY, bmax = -INFINITY, smin = INFINITY, smax = -INFINITY;
#pragma unroll 4
    for (int i = tid; i < blocks; i += blockDim.x) {
        const Pass1Partial p = partials[i];
        SL += p.SL;
        SR += p.SR;
        nL += p.nL;
        nR += p.nR;
        nf |= p.nonfinite;
        bmin = fminf(bmin, p.bmin);
        bmax = fmaxf(bmax, p.bmax);
        smin = fminf(smin, p.smin);
        smax = fmaxf(smax, p.smax);
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
    __syncthreads();
    if (lane == 0) {
        rd[0][wave] = SL;
        rd[1][wave] = SR;
        rl[0][wave] = nL;
        rl[1][wave] = nR;
        ru[wave] = nf;
        rf[0][wave] = bmin;
        rf[1][wave] = bmax;
        rf[2][wave] = smin;
        rf[3][wave] = smax;
    }
    __syncthreads();
    if (tid == 0) {
        Pass1Partial t;
        t.SL = 0.0;
        t.SR = 0.0;
        t.nL = 0;
        t.nR = 0;
        t.nonfinite = 0;
        t.bmin = INFINITY;
        t.bmax = -INFINITY;
        t.smin = INFINITY;
        t.smax = -INFINITY;
        for (int w = 0; w < nw; ++w) {
            t.SL += rd[0][w];
            t.SR += rd[1][w];
            t.nL += rl[0][w];
            t.nR += rl[1][w];
            t.nonfinite |= ru[w];
            t.bmin = fminf(t.bmin, rf[0][w]);
            t.bmax = fmaxf(t.bmax, rf[1][w]);
            t.smin = fminf(t.smin, rf[2][w]);
            t.smax = fmaxf(t.smax, rf[3][w]);
        }
        out = t;
        st->SL = t.SL;
        st->SR = t.SR;
        st->nL = t.nL;
        st->nR = t.nR;
        st->nonfinite = t.nonfinite;
        st->bmin = t.bmin;
        st->bmax = t.bmax;
        st->smin = t.smin;
        st->smax = t.smax;
    }
    __syncthreads();
    return out;
}

}  // namespace stk
