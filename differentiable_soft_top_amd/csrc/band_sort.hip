// band_sort.hip -- bucketing of the middle band (the band sort's first level).
//
// aiqbench.com abstract of Fast LapSum: with the bracket in place, only the
// scores in a thin band near the threshold are sorted; gist.science summary,
// section 2.2 step 3: the exact solver runs on that band alone.
//
// gfx950 design: a value-bucket sort whose second level runs in the solve.  The band lies in [bmin, bmax] (known
// from pass-1) and its density there is smooth, so kBuckets equal-width value
// buckets hold similar counts.  Three kernels:
//   1. histogram: per-work-group LDS bucket counts, one row per work-group;
//   2. scatter: every work-group reads all rows, forms the bucket starts and
//      its own offsets (bucket-major, work-group-minor) and moves each
//      element of its chunk to its bucket (order within a bucket is
//      arbitrary);
//   3. bucket summaries: one work-group per bucket records its count,
//      smallest and largest value and the anchored exponential sums
//      (TA = sum e^{(x-last)/alpha}, TB = sum e^{-(x-first)/alpha}) that the
//      segment solve scans.  No bucket is sorted here: the solve locates the
//      one bucket that holds the root and sorts only that one, in LDS.
// The bucket index floor((v - bmin) * kBuckets / (bmax - bmin)) is
// non-decreasing in v, so bucket order is value order.
#include "stk_common.hpp"
#include "stk_layout.hpp"
#include "stk_prof.hpp"

namespace stk {

namespace {

__device__ __forceinline__ int bucket_of(float v, double lo, double scale)
{
    const double t = ((double)v - lo) * scale;
    int b = (int)t;
    b = b < 0 ? 0 : b;
    return b > kBuckets - 1 ? kBuckets - 1 : b;
}

// Shared early-exit test: band overflow or a non-finite score makes every
// band kernel a no-op (the segment solve records why).
__device__ __forceinline__ bool band_unusable(const Status* st, int64_t cap)
{
    return st->nB > (uint64_t)cap;
}

// Elements per histogram/scatter work-group: at least kBandChunkMin, and
// enough that at most kBandGroups work-groups share the band (the scatter
// reads every group's histogram row).
__device__ __forceinline__ uint64_t band_chunk(uint64_t nB)
{
    const uint64_t c = (nB + kBandGroups - 1) / kBandGroups;
    return c < (uint64_t)kBandChunkMin ? (uint64_t)kBandChunkMin : c;
}

__device__ __forceinline__ int band_groups(uint64_t nB)
{
    return nB == 0 ? 1 : (int)((nB + band_chunk(nB) - 1) / band_chunk(nB));
}

// Bucket range: the bracket itself when both ends are finite (the band lies
// in [a_L, a_R)), else the band's own min/max from the pass-1 partials (same
// fixed-order fold in every work-group, so every work-group maps a value to
// the same bucket).
__device__ void bucket_range(const BandArgs& a, double* lo, double* scale)
{
    __shared__ float mm[2];
    const float aL = a.st->aL, aR = a.st->aR;
    float l = aL, h = aR;
    if (aL == -INFINITY || aR == INFINITY) {
        float bmin = INFINITY, bmax = -INFINITY;
        for (int i = threadIdx.x; i < a.p1_blocks; i += blockDim.x) {
            bmin = fminf(bmin, a.p1[i].bmin);
            bmax = fmaxf(bmax, a.p1[i].bmax);
        }
        bmin = wave_min(bmin);
        bmax = wave_max(bmax);
        __shared__ float wmm[2][kSortThreads / kWave];
        if ((threadIdx.x & (kWave - 1)) == 0) {
            wmm[0][threadIdx.x / kWave] = bmin;
            wmm[1][threadIdx.x / kWave] = bmax;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            float x = INFINITY, y = -INFINITY;
            for (int w = 0; w < kSortThreads / kWave; ++w) {
                x = fminf(x, wmm[0][w]);
                y = fmaxf(y, wmm[1][w]);
            }
            mm[0] = x;
            mm[1] = y;
        }
        __syncthreads();
        l = mm[0];
        h = mm[1];
    }
    *lo = l;
    *scale = (h > l) ? (double)kBuckets / ((double)h - (double)l) : 0.0;
}

}  // namespace

// Per-work-group bucket counts of one chunk of the band (no cross-group step:
// the scatter kernel derives the offsets from all rows).
__global__ __launch_bounds__(kSortThreads) void band_hist_kernel(BandArgs a)
{
    __shared__ uint32_t hist[kBuckets];
    const Status* st = a.st;
    if (band_unusable(st, a.cap))
        return;
    const uint64_t nB = st->nB;
    const int used = band_groups(nB);
    if ((int)blockIdx.x >= used)
        return;
    const int tid = threadIdx.x;
    double lo, scale;
    bucket_range(a, &lo, &scale);
    for (int i = tid; i < kBuckets; i += kSortThreads)
        hist[i] = 0;
    __syncthreads();
    const uint64_t chunk = band_chunk(nB);
    const uint64_t e0 = (uint64_t)blockIdx.x * chunk;
    const uint64_t e1 = e0 + chunk < nB ? e0 + chunk : nB;
    // eight loads in flight before the LDS atomics
    for (uint64_t ib = e0; ib < e1; ib += 8 * kSortThreads) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint64_t i = ib + (uint64_t)j * kSortThreads + tid;
            v[j] = i < e1 ? a.band[i] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint64_t i = ib + (uint64_t)j * kSortThreads + tid;
            if (i < e1)
                atomicAdd(&hist[bucket_of(v[j], lo, scale)], 1u);
        }
    }
    __syncthreads();
    uint32_t* row = a.hist + (size_t)blockIdx.x * kBuckets;
    for (int i = tid; i < kBuckets; i += kSortThreads)
        row[i] = hist[i];
}

// Each work-group reads every row of the bucket histogram, forms the bucket
// starts (exclusive scan of the column sums) and its own offsets (plus the
// counts of the groups before it), then scatters its chunk.  Work-group 0
// also publishes the bucket starts.
__global__ __launch_bounds__(kSortThreads) void band_scatter_kernel(BandArgs a)
{
    constexpr int kPer = kBuckets / kSortThreads;  // buckets per thread
    static_assert(kPer == 2, "one uint2 per thread and row");
    __shared__ uint32_t cursor[kBuckets];
    __shared__ uint32_t scan_tmp[kSortThreads / kWave];
    const Status* st = a.st;
    if (band_unusable(st, a.cap))
        return;
    const uint64_t nB = st->nB;
    const int used = band_groups(nB);
    if ((int)blockIdx.x >= used)
        return;
    const int tid = threadIdx.x;
    const int me = blockIdx.x;
    double lo, scale;
    bucket_range(a, &lo, &scale);

    uint32_t tot[kPer], before[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        tot[j] = 0;
        before[j] = 0;
    }
    // all rows' loads issued together (kBandGroups <= 128 rows)
    static_assert(kBandGroups % 16 == 0, "row batches of 16");
    for (int wb = 0; wb < used; wb += 16) {
        uint2 x[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
            x[u] = wb + u < used ? *reinterpret_cast<const uint2*>(a.hist + (size_t)(wb + u) * kBuckets + tid * kPer)
                                 : make_uint2(0u, 0u);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            tot[0] += x[u].x;
            tot[1] += x[u].y;
            before[0] += wb + u < me ? x[u].x : 0u;
            before[1] += wb + u < me ? x[u].y : 0u;
        }
    }
    uint32_t local = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        local += tot[j];
    // exclusive scan of the per-thread sums: lane shuffles, then the wave
    // totals through LDS (one barrier)
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    uint32_t incl = local;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off, kWave);
        if (lane >= off)
            incl += o;
    }
    if (lane == kWave - 1)
        scan_tmp[wave] = incl;
    __syncthreads();
    uint32_t base = incl - local;
    for (int w = 0; w < wave; ++w)
        base += scan_tmp[w];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int b = tid * kPer + j;
        cursor[b] = base + before[j];
        if (me == 0)
            a.bstart[b] = base;
        base += tot[j];
    }
    if (me == 0 && tid == 0)
        a.bstart[kBuckets] = (uint32_t)nB;
    __syncthreads();
    const uint64_t chunk = band_chunk(nB);
    const uint64_t e0 = (uint64_t)me * chunk;
    const uint64_t e1 = e0 + chunk < nB ? e0 + chunk : nB;
    for (uint64_t ib = e0; ib < e1; ib += 8 * kSortThreads) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint64_t i = ib + (uint64_t)j * kSortThreads + tid;
            v[j] = i < e1 ? a.band[i] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint64_t i = ib + (uint64_t)j * kSortThreads + tid;
            if (i < e1) {
                const uint32_t pos = atomicAdd(&cursor[bucket_of(v[j], lo, scale)], 1u);
                a.band_sorted[pos] = v[j];
            }
        }
    }
}

// Fixed-order fold of pass-1 partials [i0, i1) by the first wave; lane 0
// returns the result.
__device__ Pass1Partial fold_partials_wave(const Pass1Partial* p, int i0, int i1)
{
    const int lane = threadIdx.x & (kWave - 1);
    double SL = 0.0, SR = 0.0;
    unsigned long long nL = 0, nR = 0;
    uint32_t nf = 0;
    float bmin = INFINITY, bmax = -INFINITY, smin = INFINITY, smax = -INFINITY;
    for (int i = i0 + lane; i < i1; i += kWave) {
        const Pass1Partial q = p[i];
        SL += q.SL;
        SR += q.SR;
        nL += q.nL;
        nR += q.nR;
        nf |= q.nonfinite;
        bmin = fminf(bmin, q.bmin);
        bmax = fmaxf(bmax, q.bmax);
        smin = fminf(smin, q.smin);
        smax = fmaxf(smax, q.smax);
    }
    Pass1Partial r;
    r.SL = wave_sum(SL);
    r.SR = wave_sum(SR);
    r.nL = wave_sum_u64(nL);
    r.nR = wave_sum_u64(nR);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        nf |= __shfl_xor(nf, off, kWave);
    r.nonfinite = nf;
    r.bmin = wave_min(bmin);
    r.bmax = wave_max(bmax);
    r.smin = wave_min(smin);
    r.smax = wave_max(smax);
    return r;
}

// ---------------------------------------------------------------------------
// Order-independent sums.  A bucket's elements arrive in an order that
// depends on atomic reservations (pass-1 band appends, scatter cursors), so
// fp64 accumulation would round differently from run to run.  Each term
// (an anchored exponential, in [0, 1]) is instead cut to a multiple of 2^-64
// (truncation, a function of the term alone) and summed exactly as a 128-bit
// integer; the total is converted back to fp64 once.  The cut costs under
// 2^-64 per term, far below fp64 rounding of the sum.
// ---------------------------------------------------------------------------
struct Fix128 {
    uint64_t lo, hi;  // value = (hi * 2^64 + lo) * 2^-64
};

__device__ __forceinline__ Fix128 fix_of(double e)
{
    const uint64_t bits = (uint64_t)__double_as_longlong(e);
    const int E = (int)((bits >> 52) & 0x7FF);
    Fix128 r;
    r.lo = 0;
    r.hi = 0;
    if (E == 0 || (bits >> 63))
        return r;  // zero, subnormal (below 2^-1022) or negative: nothing
    const uint64_t mi = (bits & 0xFFFFFFFFFFFFFull) | (1ull << 52);  // e = mi * 2^(E - 1075)
    const int sh = E - 1011;                                         // e * 2^64 = mi * 2^sh
    if (sh >= 64) {
        r.hi = mi << (sh - 64);  // only for e >= 2^11, not reached for terms in [0, 1]
    } else if (sh > 0) {
        r.lo = mi << sh;
        r.hi = mi >> (64 - sh);
    } else if (sh > -64) {
        r.lo = mi >> (-sh);
    }
    return r;
}

__device__ __forceinline__ void fix_add(Fix128& a, const Fix128& b)
{
    const uint64_t lo = a.lo + b.lo;
    a.hi += b.hi + (lo < a.lo ? 1ull : 0ull);
    a.lo = lo;
}

__device__ __forceinline__ Fix128 fix_wave_sum(Fix128 v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        Fix128 o;
        o.lo = __shfl_xor(v.lo, off, kWave);
        o.hi = __shfl_xor(v.hi, off, kWave);
        fix_add(v, o);
    }
    return v;
}

__device__ __forceinline__ double fix_to_double(const Fix128& v)
{
    return (double)v.hi + ldexp((double)v.lo, -64);
}

// One work-group per bucket: the bucket's summary for the level-1 scan of the
// segment solve -- count, smallest and largest value, TA = sum e^{(x-hi)/alpha},
// TB = sum e^{-(x-lo)/alpha} -- from its unordered elements.  Only the one
// bucket that holds the root is ever sorted (by the solve, in LDS).  Each
// work-group also folds its share of the pass-1 partials, so the
// single-work-group solve reads kBuckets of them.
__global__ __launch_bounds__(kSortThreads) void bucket_agg_kernel(BandArgs a)
{
    constexpr int kHeld = 4;  // elements per thread kept in registers between the two sweeps
    __shared__ Fix128 red[2][kSortThreads / kWave];
    __shared__ float redf[2][kSortThreads / kWave];
    const Status* st = a.st;
    if (band_unusable(st, a.cap))
        return;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    if (wave == 0) {
        const int per = (a.p1_blocks + kBuckets - 1) / kBuckets;
        const int i0 = b * per < a.p1_blocks ? b * per : a.p1_blocks;
        const int i1 = i0 + per < a.p1_blocks ? i0 + per : a.p1_blocks;
        const Pass1Partial r = fold_partials_wave(a.p1, i0, i1);
        if (lane == 0)
            a.p1_super[b] = r;
    }
    const uint32_t start = a.bstart[b];
    const uint32_t cnt = a.bstart[b + 1] - start;
    GroupAgg g;
    g.cnt = cnt;
    g.start = start;
    if (cnt == 0) {
        if (tid == 0) {
            g.TA = 0.0;
            g.TB = 0.0;
            g.lo = 0.f;
            g.hi = 0.f;
            a.agg[b] = g;
        }
        return;
    }
    const float* x = a.band_sorted + start;
    // sweep 1: smallest and largest value (the anchors)
    float v[kHeld];
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kHeld; ++j) {
        const uint32_t i = (uint32_t)(j * kSortThreads + tid);
        v[j] = i < cnt ? x[i] : 0.f;
        if (i < cnt) {
            mn = fminf(mn, v[j]);
            mx = fmaxf(mx, v[j]);
        }
    }
    for (uint32_t i = kHeld * kSortThreads + tid; i < cnt; i += kSortThreads) {
        const float t = x[i];
        mn = fminf(mn, t);
        mx = fmaxf(mx, t);
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
        redf[0][wave] = mn;
        redf[1][wave] = mx;
    }
    __syncthreads();
    float lo = INFINITY, hi = -INFINITY;
    for (int w = 0; w < kSortThreads / kWave; ++w) {
        lo = fminf(lo, redf[0][w]);
        hi = fmaxf(hi, redf[1][w]);
    }
    // sweep 2: the anchored exponential sums, exact and order-independent
    const double c = a.log2e_over_alpha;
    const double dlo = lo, dhi = hi;
    Fix128 TA{0ull, 0ull}, TB{0ull, 0ull};
#pragma unroll
    for (int j = 0; j < kHeld; ++j) {
        const uint32_t i = (uint32_t)(j * kSortThreads + tid);
        if (i < cnt) {
            fix_add(TA, fix_of(exp2_nonpos(((double)v[j] - dhi) * c)));
            fix_add(TB, fix_of(exp2_nonpos((dlo - (double)v[j]) * c)));
        }
    }
    for (uint32_t i = kHeld * kSortThreads + tid; i < cnt; i += kSortThreads) {
        const double t = x[i];
        fix_add(TA, fix_of(exp2_nonpos((t - dhi) * c)));
        fix_add(TB, fix_of(exp2_nonpos((dlo - t) * c)));
    }
    TA = fix_wave_sum(TA);
    TB = fix_wave_sum(TB);
    if (lane == 0) {
        red[0][wave] = TA;
        red[1][wave] = TB;
    }
    __syncthreads();
    if (tid == 0) {
        Fix128 sa{0ull, 0ull}, sb{0ull, 0ull};
        for (int w = 0; w < kSortThreads / kWave; ++w) {
            fix_add(sa, red[0][w]);
            fix_add(sb, red[1][w]);
        }
        g.TA = fix_to_double(sa);
        g.TB = fix_to_double(sb);
        g.lo = lo;
        g.hi = hi;
        a.agg[b] = g;
    }
}

hipError_t launch_band_sort(const BandArgs& a, hipStream_t stream)
{
    STK_LAUNCH(kKBandHist, stream, band_hist_kernel, dim3(a.blocks), dim3(kSortThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    STK_LAUNCH(kKBandScatter, stream, band_scatter_kernel, dim3(a.blocks), dim3(kSortThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    STK_LAUNCH(kKBucketAgg, stream, bucket_agg_kernel, dim3(kBuckets), dim3(kSortThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace stk
