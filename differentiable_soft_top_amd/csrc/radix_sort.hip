// radix_sort.hip -- full device sort for the worst-case route.
//
// aiqbench.com abstract of Fast LapSum: a full-sort fallback covers the worst
// case of the bracketed solver.  This is a least-significant-digit radix
// sort of all n scores on their order-preserving u32 keys, offset by the
// smallest key so only the digits that vary are sorted (8-bit digits).
//
// Per digit, reduce-then-scan with two kernels:
//   upsweep   -- each work-group histograms the digit of its 8192-key tile;
//                the last work-group to finish turns the [digit][tile]
//                histogram into exclusive global offsets;
//   downsweep -- each work-group ranks its tile's keys stably (wave-level
//                match by eight ballots, wave counts combined in LDS in
//                (round, wave, lane) order, i.e. index order) and writes
//                each key to offset[digit][tile] + rank.
// Stability of every pass makes the LSD sort correct for any ties (the
// clustered workload is 60% one value).
#include "stk_common.hpp"
#include "stk_layout.hpp"
#include "stk_prof.hpp"

namespace stk {

namespace {

struct PassArgs {
    const float* s;        // pass 0 input
    const uint32_t* in;    // later passes
    uint32_t* out;
    uint32_t* hist;        // [kRadixBins][gp]
    int64_t n;
    int32_t g;             // tiles
    int32_t gp;            // row stride of hist (g rounded up to 4)
    uint32_t key_min;
    int32_t shift;
    Status* st;
};

template <bool kFromFloat>
__device__ __forceinline__ uint32_t load_key(const PassArgs& a, int64_t i)
{
    if (kFromFloat)
        return float_to_key(a.s[i]) - a.key_min;
    return a.in[i];
}

// Lanes of this wave whose digit equals mine (among lanes with valid=true).
__device__ __forceinline__ uint64_t match_digit(uint32_t d, bool valid)
{
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const bool bit = (d >> b) & 1u;
        const uint64_t bb = __ballot(bit);
        peers &= bit ? bb : ~bb;
    }
    return peers;
}

}  // namespace

template <bool kFromFloat>
__global__ __launch_bounds__(kRadixThreads) void radix_upsweep(PassArgs a)
{
    __shared__ uint32_t hist[kRadixBins];
    __shared__ uint32_t tot[kRadixBins];
    __shared__ uint32_t is_last;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    for (int i = tid; i < kRadixBins; i += kRadixThreads)
        hist[i] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kRadixTile;
    for (int r = 0; r < kRadixKeysPerThread; ++r) {
        const int64_t i = base + (int64_t)r * kRadixThreads + tid;
        const bool valid = i < a.n;
        const uint32_t key = valid ? load_key<kFromFloat>(a, i) : 0u;
        const uint32_t d = (key >> a.shift) & 0xFFu;
        const uint64_t peers = match_digit(d, valid);
        if (valid && lane == __ffsll((long long)peers) - 1)
            atomicAdd(&hist[d], (uint32_t)__popcll(peers));
    }
    __syncthreads();
    for (int dgt = tid; dgt < kRadixBins; dgt += kRadixThreads)
        a.hist[(size_t)dgt * a.gp + blockIdx.x] = hist[dgt];
    __syncthreads();
    if (tid == 0) {
        fence_agent();
        const uint32_t t = atomicAdd(&a.st->ticket_radix, 1u);
        is_last = t == (uint32_t)(a.g - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (!is_last)
        return;
    fence_agent();

    // last work-group: thread d owns digit row d of the histogram
    static_assert(kRadixThreads == kRadixBins, "one thread per digit");
    const int dgt = tid;
    uint32_t* row = a.hist + (size_t)dgt * a.gp;
    uint32_t total = 0;
    for (int t = 0; t < a.g; t += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + t);
        total += v.x + (t + 1 < a.g ? v.y : 0u) + (t + 2 < a.g ? v.z : 0u) + (t + 3 < a.g ? v.w : 0u);
    }
    tot[dgt] = total;
    __syncthreads();
    for (int off = 1; off < kRadixBins; off <<= 1) {
        const uint32_t v = dgt >= off ? tot[dgt - off] : 0u;
        __syncthreads();
        tot[dgt] += v;
        __syncthreads();
    }
    uint32_t run = tot[dgt] - total;  // exclusive digit base
    for (int t = 0; t < a.g; t += 4) {
        uint4 v = *reinterpret_cast<const uint4*>(row + t);
        uint4 o;
        o.x = run;
        run += v.x;
        o.y = run;
        run += (t + 1 < a.g) ? v.y : 0u;
        o.z = run;
        run += (t + 2 < a.g) ? v.z : 0u;
        o.w = run;
        run += (t + 3 < a.g) ? v.w : 0u;
        *reinterpret_cast<uint4*>(row + t) = o;
    }
    if (tid == 0)
        a.st->ticket_radix = 0;
}

template <bool kFromFloat>
__global__ __launch_bounds__(kRadixThreads) void radix_downsweep(PassArgs a)
{
    constexpr int kWaves = kRadixThreads / kWave;
    __shared__ uint32_t goff[kRadixBins];
    __shared__ uint32_t running[kRadixBins];
    __shared__ uint32_t wcnt[kWaves][kRadixBins];
    __shared__ uint32_t wpre[kWaves][kRadixBins];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    for (int d = tid; d < kRadixBins; d += kRadixThreads) {
        goff[d] = a.hist[(size_t)d * a.gp + blockIdx.x];
        running[d] = 0;
        for (int w = 0; w < kWaves; ++w)
            wcnt[w][d] = 0;
    }
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kRadixTile;
    for (int r = 0; r < kRadixKeysPerThread; ++r) {
        const int64_t i = base + (int64_t)r * kRadixThreads + tid;
        const bool valid = i < a.n;
        const uint32_t key = valid ? load_key<kFromFloat>(a, i) : 0u;
        const uint32_t d = (key >> a.shift) & 0xFFu;
        const uint64_t peers = match_digit(d, valid);
        const uint32_t rank = rank_in_mask(peers);
        if (valid && rank == 0)
            wcnt[wave][d] = (uint32_t)__popcll(peers);
        __syncthreads();
        for (int dd = tid; dd < kRadixBins; dd += kRadixThreads) {
            uint32_t run = running[dd];
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                wpre[w][dd] = run;
                run += wcnt[w][dd];
                wcnt[w][dd] = 0;
            }
            running[dd] = run;
        }
        __syncthreads();
        if (valid)
            a.out[goff[d] + wpre[wave][d] + rank] = key;
    }
}

hipError_t launch_radix_sort(const RadixArgs& ra, hipStream_t stream)
{
    PassArgs a;
    a.s = ra.s;
    a.n = ra.n;
    a.g = ra.g_radix;
    a.gp = (ra.g_radix + 3) & ~3;
    a.hist = ra.hist;
    a.key_min = ra.key_min;
    a.st = ra.st;
    uint32_t* bufs[2] = {ra.keys0, ra.keys1};
    for (int p = 0; p < ra.passes; ++p) {
        a.shift = 8 * p;
        a.in = p == 0 ? nullptr : bufs[(p - 1) & 1];
        a.out = bufs[p & 1];
        if (p == 0) {
            STK_LAUNCH(kKRadixUp, stream, radix_upsweep<true>, dim3(a.g), dim3(kRadixThreads), 0, stream, a);
            STK_LAUNCH(kKRadixDown, stream, radix_downsweep<true>, dim3(a.g), dim3(kRadixThreads), 0, stream, a);
        } else {
            STK_LAUNCH(kKRadixUp, stream, radix_upsweep<false>, dim3(a.g), dim3(kRadixThreads), 0, stream, a);
            STK_LAUNCH(kKRadixDown, stream, radix_downsweep<false>, dim3(a.g), dim3(kRadixThreads), 0, stream, a);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (ra.sorted_out)
        *ra.sorted_out = bufs[(ra.passes - 1) & 1];
    return hipSuccess;
}

}  // namespace stk
