// stk_common.hpp -- device helpers shared by the soft top-k kernels (gfx950).
//
// Nothing here is specific to one kernel: the fp64 exponential used wherever
// a sum of exponentials feeds the threshold, the order-preserving fp32 key,
// the Philox4x32-10 counter-based generator, wave-64 reductions and a
// work-group bitonic sort of keys held in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace stk {

constexpr int kWave = 64;
constexpr double kLog2e = 1.4426950408889634;
constexpr double kLn2 = 0.6931471805599453;

// ---------------------------------------------------------------------------
// 2^y for y <= 0 in fp64, relative error ~2e-16.
// Range reduction y = j + r with j = rint(y), |r| <= 1/2, then
// e^(r ln 2) by its Taylor series to degree 12 (the truncation term
// (ln2/2)^13/13! is below 2e-16), then an exact scaling by 2^j.
// Arguments below -1100 (and NaN) give 0.  Every exponential whose error
// reaches the threshold goes through this function: the hardware fp32
// exponential is accurate to ~1e-7, which summed over ~1e5 near-threshold
// terms could move the selected mass by more than 1e-3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double exp2_nonpos(double y)
{
    y = fmax(y, -1100.0);          // fmax(NaN, c) = c
    y = fmin(y, 0.0);
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

// The same function with the polynomial in Estrin's scheme: a few more
// operations but a dependency depth of 5 instead of 13, for chains of
// dependent exponentials (scans) where latency, not throughput, decides.
__device__ __forceinline__ double exp2_nonpos_lowdepth(double y)
{
    y = fmax(y, -1100.0);
    y = fmin(y, 0.0);
    const double j = __builtin_rint(y);
    const double t = (y - j) * kLn2;
    const double t2 = t * t;
    const double t4 = t2 * t2;
    const double t8 = t4 * t4;
    const double q01 = fma(t, 1.0, 1.0);
    const double q23 = fma(t, 0.16666666666666666, 0.5);
    const double q45 = fma(t, 0.008333333333333333, 0.041666666666666664);
    const double q67 = fma(t, 0.0001984126984126984, 0.001388888888888889);
    const double q89 = fma(t, 2.7557319223985893e-06, 2.48015873015873e-05);
    const double qab = fma(t, 2.505210838544172e-08, 2.755731922398589e-07);
    const double r0 = fma(q23, t2, q01);
    const double r1 = fma(q67, t2, q45);
    const double r2 = fma(qab, t2, q89);
    const double s0 = fma(r1, t4, r0);
    const double s1 = fma(2.08767569878681e-09, t4, r2);
    return ldexp(fma(s1, t8, s0), (int)j);
}

// e^(x/alpha) for x <= 0 given inv = log2(e)/alpha.
__device__ __forceinline__ double exp_scaled_nonpos(double x, double log2e_over_alpha)
{
    return exp2_nonpos(x * log2e_over_alpha);
}

// ---------------------------------------------------------------------------
// Order-preserving map fp32 -> u32 (after folding -0 into +0, so the band
// test a_L <= v and the key order agree).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t float_to_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k)
{
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ bool is_nonfinite(float v)
{
    return (__float_as_uint(v) & 0x7f800000u) == 0x7f800000u;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64 multiplies with the
// published multipliers and Weyl key increments.
// ---------------------------------------------------------------------------
struct Philox4 {
    uint32_t v[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t lo0 = 0xD2511F53u * c0;
        const uint32_t hi0 = __umulhi(0xD2511F53u, c0);
        const uint32_t lo1 = 0xCD9E8D57u * c2;
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2);
        const uint32_t n0 = hi1 ^ c1 ^ k0;
        const uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    Philox4 out;
    out.v[0] = c0;
    out.v[1] = c1;
    out.v[2] = c2;
    out.v[3] = c3;
    return out;
}

// ---------------------------------------------------------------------------
// The VJP's g - G/D with the fp64 ratio carried as an unevaluated float pair
// hi + lo.  Where g nearly cancels the ratio (one density dominating D, a
// saturated row) g - hi is exact (the operands are within a factor of two),
// so the small difference keeps its relative accuracy; a plain fp32 ratio
// would leave an error of half its ulp there.  A non-finite ratio (a
// non-finite g somewhere) passes through hi.
// ---------------------------------------------------------------------------
struct Ratio2 {
    float hi, lo;
};

__device__ __forceinline__ Ratio2 split_ratio(double r)
{
    Ratio2 q;
    q.hi = (float)r;
    q.lo = isfinite(q.hi) ? (float)(r - (double)q.hi) : 0.0f;
    return q;
}

__device__ __forceinline__ float minus_ratio(float g, Ratio2 q) { return (g - q.hi) - q.lo; }

// D += d, G += g d in fp64 (the product of two floats is exact there).  The
// ratio G/D is then off by fp64 rounding only, and the fp32 error of each d
// moves it by a relative fp32 ulp of (g_i - G/D) d_i / D, never of G/D.
__device__ __forceinline__ void acc_dg(float d, float g, double& D, double& G)
{
    D += (double)d;
    G = fma((double)g, (double)d, G);
}

// ---------------------------------------------------------------------------
// Wave-64 reductions (every lane receives the result; butterfly order is
// fixed, so results are bitwise reproducible).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float wave_min(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = fminf(v, __shfl_xor(v, off, kWave));
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of active lanes below this one in `mask`.
__device__ __forceinline__ uint32_t rank_in_mask(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// ---------------------------------------------------------------------------
// Two order statistics of the first cnt of kThreads * R u32 keys held R per
// thread in blocked order (position t*R + r; the values in any order; keys
// at positions >= cnt are ignored), without sorting: most-significant-digit
// radix selection on the offsets key - min, 8 bits a round, from the highest
// bit in which the offsets differ (so bits that every key shares cost no
// round, and the first digit already spreads keys drawn from a narrow
// range).  Each round counts, among the keys that share the digits chosen
// so far for a target, how many carry each value of the next digit (LDS
// atomics); one wave per target scans the 256 counts and keeps the digit
// whose count range holds the target's remaining rank.  Both targets run
// together (their prefixes may differ); a round costs two barriers, the two
// 512-word histogram buffers alternating so that clearing the next round's
// buffer never races with the scan of the current one.
//   r0, r1 -- 1-based ranks; one outside [1, cnt] leaves its output untouched.
//   hist   -- LDS, 2 * 512 words, 16-byte aligned;  state -- LDS, 4 + 2 *
//             (kThreads / 64) words;  out -- 2 words.
// Every thread of the work-group must call it; out is valid after it returns.
// ---------------------------------------------------------------------------
template <int kThreads, int R>
__device__ __forceinline__ void block_select2(const uint32_t (&v)[R], int cnt, int64_t r0, int64_t r1, uint32_t* hist,
                                              uint32_t* state, uint32_t* out)
{
    static_assert(kThreads >= 128, "one wave per target");
    constexpr int kW = kThreads / kWave;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const bool want0 = r0 >= 1 && r0 <= (int64_t)cnt;
    const bool want1 = r1 >= 1 && r1 <= (int64_t)cnt;
    // ---- smallest and largest key ------------------------------------------
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (tid * R + r < cnt) {
            mn = min(mn, v[r]);
            mx = max(mx, v[r]);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor(mn, off, kWave));
        mx = max(mx, (uint32_t)__shfl_xor(mx, off, kWave));
    }
    uint32_t* wmn = state + 4;
    uint32_t* wmx = state + 4 + kW;
    if (lane == 0) {
        wmn[wave] = mn;
        wmx[wave] = mx;
    }
    if (tid == 0) {
        state[0] = 0u;  // offset digits chosen so far, target 0 / 1
        state[1] = 0u;
        state[2] = want0 ? (uint32_t)r0 : 1u;  // rank among the keys with those digits
        state[3] = want1 ? (uint32_t)r1 : 1u;
    }
    __syncthreads();
    mn = 0xFFFFFFFFu;
    mx = 0u;
    for (int w = 0; w < kW; ++w) {
        mn = min(mn, wmn[w]);
        mx = max(mx, wmx[w]);
    }
    const uint32_t span = mx >= mn ? mx - mn : 0u;  // cnt == 0 leaves mn > mx
    const int bits = span ? 32 - __builtin_clz(span) : 0;
    const int rounds = (bits + 7) / 8;
    uint32_t mask = 0u;
    for (int round = 0; round < rounds; ++round) {
        const int shift = bits - 8 * (round + 1) > 0 ? bits - 8 * (round + 1) : 0;
        uint32_t* h = hist + (round & 1) * 512;
        for (int i = tid; i < 512; i += kThreads)
            h[i] = 0u;
        __syncthreads();  // cleared; state of the previous round visible
        const uint32_t p0 = state[0], p1 = state[1];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (tid * R + r < cnt) {
                const uint32_t o = v[r] - mn;
                const uint32_t d = (o >> shift) & 255u;
                if ((o & mask) == p0)
                    atomicAdd(&h[d], 1u);
                if ((o & mask) == p1)
                    atomicAdd(&h[256 + d], 1u);
            }
        }
        __syncthreads();  // counts complete
        if (wave < 2) {
            const uint4 c = *reinterpret_cast<const uint4*>(h + 256 * wave + 4 * lane);
            const uint32_t loc = c.x + c.y + c.z + c.w;
            uint32_t incl = loc;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const uint32_t o = __shfl_up(incl, off, kWave);
                if (lane >= off)
                    incl += o;
            }
            const uint32_t before = incl - loc;
            const uint32_t rem = state[2 + wave];
            if (rem > before && rem <= incl) {
                uint32_t d = 4u * (uint32_t)lane, cum = before;
                if (rem > cum + c.x) {
                    cum += c.x;
                    ++d;
                    if (rem > cum + c.y) {
                        cum += c.y;
                        ++d;
                        if (rem > cum + c.z) {
                            cum += c.z;
                            ++d;
                        }
                    }
                }
                state[wave] |= d << shift;
                state[2 + wave] = rem - cum;
            }
        }
        // the digits below `shift` stay unchosen; a short last round (bits
        // not a multiple of 8) overlaps the previous one, whose digits then
        // match on the overlap by construction
        mask |= 255u << shift;
    }
    __syncthreads();
    if (tid == 0) {
        if (want0)
            out[0] = mn + state[0];
        if (want1)
            out[1] = mn + state[1];
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Ascending bitonic network over N keys held in registers.  Stages are
// template parameters, so every register index is a compile-time constant
// (nested runtime-bounded loops would leave the unroller a variable trip
// count and the array in scratch memory).
// ---------------------------------------------------------------------------
template <int N, int K, int J>
struct RegBitonicStage {
    static __device__ __forceinline__ void run(uint32_t (&a)[N])
    {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int l = i ^ J;
            if (l > i) {
                const uint32_t x = a[i], y = a[l];
                const bool up = (i & K) == 0;
                a[i] = up ? min(x, y) : max(x, y);
                a[l] = up ? max(x, y) : min(x, y);
            }
        }
        RegBitonicStage<N, K, J / 2>::run(a);
    }
};

template <int N, int K>
struct RegBitonicStage<N, K, 0> {
    static __device__ __forceinline__ void run(uint32_t (&)[N]) {}
};

template <int N, int K, bool kDone = (K > N)>
struct RegBitonicLevel {
    static __device__ __forceinline__ void run(uint32_t (&a)[N])
    {
        RegBitonicStage<N, K, K / 2>::run(a);
        RegBitonicLevel<N, 2 * K>::run(a);
    }
};

template <int N, int K>
struct RegBitonicLevel<N, K, true> {
    static __device__ __forceinline__ void run(uint32_t (&)[N]) {}
};

template <int N>
__device__ __forceinline__ void reg_bitonic(uint32_t (&a)[N])
{
    static_assert((N & (N - 1)) == 0, "power-of-two network");
    RegBitonicLevel<N, 2>::run(a);
}

template <int N>
__device__ __forceinline__ void sort_run(uint32_t* p, int c)
{
    uint32_t a[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
        a[i] = i < c ? p[i] : 0xFFFFFFFFu;
    reg_bitonic<N>(a);
#pragma unroll
    for (int i = 0; i < N; ++i)
        if (i < c)
            p[i] = a[i];
}

// ---------------------------------------------------------------------------
// Ascending sort of the first cnt of kThreads * R keys (held R per thread in
// blocked order; positions >= cnt ignored) into keys[0 .. cnt), by buckets:
// kThreads * B equal-width buckets over the offsets key - min (B = R / 4,
// at least 1: about four keys a bucket when the keys fill their slots),
// counted and scattered with LDS atomics; then each thread sorts its own B
// buckets in registers (a bitonic network of 8 or 16 keys, the smaller one
// when it holds the fullest bucket).  Suited to keys spread evenly over
// their range (a band of scores around the threshold).  Returns false when
// some bucket holds more than 16 keys; keys[] then holds them in bucket
// order only and the caller sorts another way.
//   scratch -- LDS, 2 * kThreads * B + 2 * (kThreads / 64) words.
// Every thread of the work-group must call it; keys[] is complete when it
// returns true.
// ---------------------------------------------------------------------------
template <int R>
constexpr int bucket_sort_per_thread() { return R / 4 > 1 ? R / 4 : 1; }

template <int kThreads, int R>
__device__ __forceinline__ bool block_bucket_sort(const uint32_t (&v)[R], int cnt, uint32_t* keys, uint32_t* scratch)
{
    static_assert((kThreads & (kThreads - 1)) == 0, "power-of-two thread count");
    constexpr int B = bucket_sort_per_thread<R>();
    static_assert((B & (B - 1)) == 0, "power-of-two buckets per thread");
    constexpr int kNB = kThreads * B;
    constexpr int kW = kThreads / kWave;
    uint32_t* bcnt = scratch;
    uint32_t* cur = scratch + kNB;
    uint32_t* wred = scratch + 2 * kNB;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (tid * R + r < cnt) {
            mn = min(mn, v[r]);
            mx = max(mx, v[r]);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor(mn, off, kWave));
        mx = max(mx, (uint32_t)__shfl_xor(mx, off, kWave));
    }
    if (lane == 0) {
        wred[wave] = mn;
        wred[kW + wave] = mx;
    }
    __syncthreads();
    mn = 0xFFFFFFFFu;
    mx = 0u;
    for (int w = 0; w < kW; ++w) {
        mn = min(mn, wred[w]);
        mx = max(mx, wred[kW + w]);
    }
    // bucket = floor(offset * kNB / (span + 1)) through a 32.32 fixed-point
    // reciprocal rounded down: non-decreasing in the offset, below kNB, and
    // the whole range of buckets in use
    const uint32_t span = mx >= mn ? mx - mn : 0u;
    const uint64_t inv = ((uint64_t)kNB << 32) / ((uint64_t)span + 1u);
    auto bucket = [&](uint32_t key) { return (uint32_t)(((uint64_t)(key - mn) * inv) >> 32); };
#pragma unroll
    for (int j = 0; j < B; ++j)
        bcnt[tid * B + j] = 0u;
    __syncthreads();  // counters cleared; every read of wred done
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (tid * R + r < cnt)
            atomicAdd(&bcnt[bucket(v[r])], 1u);
    __syncthreads();
    uint32_t c[B];
    uint32_t loc = 0u, cmax = 0u;
#pragma unroll
    for (int j = 0; j < B; ++j) {
        c[j] = bcnt[tid * B + j];
        loc += c[j];
        cmax = max(cmax, c[j]);
    }
    uint32_t incl = loc;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off, kWave);
        if (lane >= off)
            incl += o;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        cmax = max(cmax, (uint32_t)__shfl_xor(cmax, off, kWave));
    if (lane == kWave - 1)
        wred[wave] = incl;
    if (lane == 0)
        wred[kW + wave] = cmax;
    __syncthreads();
    uint32_t start = incl - loc;
    cmax = 0u;
    for (int w = 0; w < kW; ++w) {
        start += w < wave ? wred[w] : 0u;
        cmax = max(cmax, wred[kW + w]);
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
        cur[tid * B + j] = start;
        start += c[j];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (tid * R + r < cnt) {
            const uint32_t pos = atomicAdd(&cur[bucket(v[r])], 1u);
            keys[pos] = v[r];
        }
    }
    __syncthreads();
    if (cmax > 16u)
        return false;
    // this thread's buckets, one at a time (after the scatter each cursor
    // stands at its bucket's end)
#pragma unroll 1
    for (int j = 0; j < B; ++j) {
        const uint32_t cj = bcnt[tid * B + j];
        uint32_t* run = keys + (cur[tid * B + j] - cj);
        if (cmax <= 8u)
            sort_run<8>(run, (int)cj);
        else
            sort_run<16>(run, (int)cj);
    }
    __syncthreads();
    return true;
}

// ---------------------------------------------------------------------------
// Ascending sort of kThreads * R u32 keys held R per thread in blocked order
// (thread t holds positions t*R .. t*R+R-1) by a work-group of kThreads.
// Bitonic network: partners inside a thread are exchanged in registers,
// partners inside a wave by lane shuffles, partners in other waves through
// LDS (buf0 / buf1, each kThreads * R keys, alternate; one barrier per such
// stage).  Every stage index is a compile-time constant.  The caller
// synchronises before reusing buf0 / buf1.
// ---------------------------------------------------------------------------
template <int kThreads, int R>
__device__ __forceinline__ void block_bitonic_regs(uint32_t (&v)[R], uint32_t* buf0, uint32_t* buf1)
{
    constexpr int n2 = kThreads * R;
    const int tid = threadIdx.x;
    int flip = 0;
#pragma unroll
    for (int k = 2; k <= n2; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j < R) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int p = r ^ j;
                    if (p > r) {
                        const bool up = ((tid * R + r) & k) == 0;
                        const uint32_t a = v[r], b = v[p];
                        const bool sw = (a > b) == up;
                        v[r] = sw ? b : a;
                        v[p] = sw ? a : b;
                    }
                }
            } else if (j < kWave * R) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int i = tid * R + r;
                    const uint32_t o = (uint32_t)__shfl_xor((int)v[r], j / R, kWave);
                    const bool take_min = ((i & j) == 0) == ((i & k) == 0);
                    v[r] = take_min ? (v[r] < o ? v[r] : o) : (v[r] > o ? v[r] : o);
                }
            } else {
                uint32_t* buf = flip ? buf1 : buf0;
                flip ^= 1;
#pragma unroll
                for (int r = 0; r < R; ++r)
                    buf[tid * R + r] = v[r];
                __syncthreads();
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int i = tid * R + r;
                    const uint32_t o = buf[i ^ j];
                    const bool take_min = ((i & j) == 0) == ((i & k) == 0);
                    v[r] = take_min ? (v[r] < o ? v[r] : o) : (v[r] > o ? v[r] : o);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 16-byte store, optionally non-temporal (streaming outputs of large vectors:
// keeps them from crowding the caches ahead of the next pass's reads).
// ---------------------------------------------------------------------------
typedef float stk_f4v __attribute__((ext_vector_type(4)));

template <bool kNT>
__device__ __forceinline__ void store4(float4* p, float4 v)
{
    if (kNT) {
        stk_f4v w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<stk_f4v*>(p));
    } else {
        *p = v;
    }
}

// ---------------------------------------------------------------------------
// Release/acquire around "last work-group finishes the reduction" tickets.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void fence_agent() { __threadfence(); }

}  // namespace stk
