// radix_sort.hip -- full device sort for the worst-case route.
//
// aiqbench.com abstract of Fast LapSum: a full-sort fallback covers the worst
// case of the bracketed solver.  This is a least-significant-digit radix
// sort of all n scores on their order-preserving u32 keys, offset by the
// smallest key so only the digits that vary are sorted (8-bit digits).
//
// Per digit, reduce-then-scan:
//   upsweep   -- each work-group histograms the digit of its 8192-key tile
//                into the [digit][tile] histogram;
//   rowsum, rowscan -- one work-group per digit value: the row's total,
//                then the row turned into exclusive global offsets (digit
//                base from the totals of the smaller digits);
//   downsweep -- each work-group ranks its tile's keys stably (wave-level
//                match by eight ballots, wave counts combined in LDS in
//                (round, wave, lane) order, i.e. index order) into LDS in
//                destination order, then writes each digit's run to
//                offset[digit][tile] onwards.
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
}

// One work-group per digit: its count over all tiles, into the totals row
// that follows the [digit][tile] histogram.
__global__ __launch_bounds__(kRadixThreads) void radix_rowsum(PassArgs a)
{
    __shared__ uint32_t red[kRadixThreads / kWave];
    const int tid = threadIdx.x;
    const uint32_t* row = a.hist + (size_t)blockIdx.x * a.gp;
    uint32_t s = 0;
    for (int t = tid; t < a.g; t += kRadixThreads)
        s += row[t];
    s = wave_sum_u32(s);
    if ((tid & (kWave - 1)) == 0)
        red[tid / kWave] = s;
    __syncthreads();
    if (tid == 0) {
        uint32_t tot = 0;
        for (int w = 0; w < kRadixThreads / kWave; ++w)
            tot += red[w];
        a.hist[(size_t)kRadixBins * a.gp + blockIdx.x] = tot;
    }
}

// One work-group per digit: the row's counts become exclusive global offsets
// (all smaller digits first, then this digit's tiles in order).  Thread t
// owns a contiguous run of tiles; one work-group scan joins the runs.
__global__ __launch_bounds__(kRadixThreads) void radix_rowscan(PassArgs a)
{
    constexpr int kW = kRadixThreads / kWave;
    __shared__ uint32_t wsum[kW];
    __shared__ uint32_t base_sh;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int d = blockIdx.x;
    const uint32_t* tot = a.hist + (size_t)kRadixBins * a.gp;
    if (wave == 0) {
        uint32_t s = 0;
        for (int j = lane; j < d; j += kWave)
            s += tot[j];
        s = wave_sum_u32(s);
        if (lane == 0)
            base_sh = s;
    }
    uint32_t* row = a.hist + (size_t)d * a.gp;
    const int per = (a.g + kRadixThreads - 1) / kRadixThreads;
    const int t0 = tid * per < a.g ? tid * per : a.g;
    const int t1 = t0 + per < a.g ? t0 + per : a.g;
    uint32_t mine = 0;
    for (int t = t0; t < t1; ++t)
        mine += row[t];
    uint32_t incl = mine;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off, kWave);
        if (lane >= off)
            incl += o;
    }
    if (lane == kWave - 1)
        wsum[wave] = incl;
    __syncthreads();
    uint32_t run = base_sh + incl - mine;
    for (int w = 0; w < wave; ++w)
        run += wsum[w];
    for (int t = t0; t < t1; ++t) {
        const uint32_t v = row[t];
        row[t] = run;
        run += v;
    }
}

// The tile's keys are ranked stably into LDS in destination order (each
// digit's run in index order), then written out run by run, so the global
// stores go to consecutive addresses instead of 256 scattered buckets.  A
// digit's count in this tile is the step from its offset to the next
// tile's (or, for the last tile, to the next digit's first offset).
template <bool kFromFloat>
__global__ __launch_bounds__(kRadixThreads) void radix_downsweep(PassArgs a)
{
    constexpr int kWaves = kRadixThreads / kWave;
    __shared__ uint32_t goff[kRadixBins];
    __shared__ uint32_t lstart[kRadixBins];
    __shared__ uint32_t running[kRadixBins];
    __shared__ uint32_t wcnt[kWaves][kRadixBins];
    __shared__ uint32_t wpre[kWaves][kRadixBins];
    __shared__ uint32_t stage[kRadixTile];
    __shared__ uint32_t wsum[kWaves];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int t = blockIdx.x;
    static_assert(kRadixThreads == kRadixBins, "one thread per digit");
    {
        // this thread's digit: global offset and count in this tile
        const int d = tid;
        const uint32_t off = a.hist[(size_t)d * a.gp + t];
        uint32_t next;
        if (t + 1 < a.g)
            next = a.hist[(size_t)d * a.gp + t + 1];
        else if (d + 1 < kRadixBins)
            next = a.hist[(size_t)(d + 1) * a.gp];
        else
            next = (uint32_t)a.n;
        const uint32_t cnt = next - off;
        goff[d] = off;
        running[d] = 0;
        for (int w = 0; w < kWaves; ++w)
            wcnt[w][d] = 0;
        // exclusive scan of the counts over digits: the runs' starts in LDS
        uint32_t incl = cnt;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const uint32_t v = __shfl_up(incl, o, kWave);
            if (lane >= o)
                incl += v;
        }
        if (lane == kWave - 1)
            wsum[wave] = incl;
        __syncthreads();
        uint32_t ex = incl - cnt;
        for (int w = 0; w < wave; ++w)
            ex += wsum[w];
        lstart[d] = ex;
    }
    __syncthreads();
    const int64_t base = (int64_t)t * kRadixTile;
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
            stage[lstart[d] + wpre[wave][d] + rank] = key;
    }
    __syncthreads();
    const int64_t left = a.n - base;
    const int cnt = left < (int64_t)kRadixTile ? (int)left : kRadixTile;
    for (int j = tid; j < cnt; j += kRadixThreads) {
        const uint32_t key = stage[j];
        const uint32_t d = (key >> a.shift) & 0xFFu;
        a.out[goff[d] + (uint32_t)j - lstart[d]] = key;
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
        } else {
            STK_LAUNCH(kKRadixUp, stream, radix_upsweep<false>, dim3(a.g), dim3(kRadixThreads), 0, stream, a);
        }
        STK_LAUNCH(kKRadixScan, stream, radix_rowsum, dim3(kRadixBins), dim3(kRadixThreads), 0, stream, a);
        STK_LAUNCH(kKRadixScan, stream, radix_rowscan, dim3(kRadixBins), dim3(kRadixThreads), 0, stream, a);
        if (p == 0) {
            STK_LAUNCH(kKRadixDown, stream, radix_downsweep<true>, dim3(a.g), dim3(kRadixThreads), 0, stream, a);
        } else {
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
