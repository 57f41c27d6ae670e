// radix_sort.hip -- full device sort for the worst-case route.
//
// aiqbench.com abstract of Fast LapSum: a full-sort fallback covers the worst
// case of the bracketed solver.  This is a least-significant-digit radix
// sort of all n scores on their order-preserving u32 keys, offset by the
// smallest key so only the digits that vary are sorted (8-bit digits).
//
// Per digit, reduce-then-scan:
//   upsweep   -- each work-group histograms the digit of its 8192-key tile
//                into its row of the [tile][digit] counts (every key loaded
//                before any is counted; one LDS add per key into one of
//                16 sub-histograms; one coalesced 1 KiB store);
//   chunk sums, chunk scan -- the counts become exclusive global offsets
//                (digit base from the totals of the smaller digits, then
//                the tiles in order): one work-group per chunk of tiles
//                sums its rows per digit; then every chunk's work-group
//                takes its prefix and the digit bases from those sums and
//                rewrites its rows as offsets (all reads and writes are
//                whole rows);
//   downsweep -- wave w of a work-group ranks keys w*2048 ... w*2048 + 2047
//                of its tile, 64 at a time in index order: a key's rank
//                is its wave's running count of its digit plus the lanes
//                below it with the same digit (eight ballots); the running
//                counts live in the wave's own LDS row, so the 32 rounds
//                need no barrier.  One barrier later the rows become each
//                digit's prefix over the waves, the keys go to LDS in
//                destination order, and each digit's run is written to
//                its offset for this tile onwards.
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
    uint32_t* hist;        // [g][kRadixBins] counts, then offsets
    uint32_t* csum;        // [chunks][kRadixBins] chunk sums
    int64_t n;
    int32_t g;             // tiles
    int32_t chunk;         // tiles per chunk
    int32_t chunks;
    uint32_t key_min;
    int32_t shift;
    Status* st;
};


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

constexpr int kRadixWaves = kRadixThreads / kWave;
constexpr int kWaveKeys = kRadixTile / kRadixWaves;  // 2048 consecutive keys per wave
static_assert(kWaveKeys == kRadixKeysPerThread * kWave, "one key per lane per round");

// Key j (0..kRadixKeysPerThread-1) of this lane: wave-contiguous, so every
// round of a wave reads 64 consecutive keys.
__device__ __forceinline__ int64_t key_index(int64_t base, int wave, int lane, int j)
{
    return base + (int64_t)wave * kWaveKeys + (int64_t)j * kWave + lane;
}

// The tile's keys of this lane: every load is issued before any key is
// formed, and no branch sits around a load, so none waits for the one
// before it (in the last, partial tile a load of the last key stands in
// past n).
template <bool kFromFloat>
__device__ __forceinline__ void load_keys(const PassArgs& a, int64_t base, int wave, int lane,
                                          uint32_t (&key)[kRadixKeysPerThread])
{
    if (base + kRadixTile <= a.n) {
        const int64_t i0 = key_index(base, wave, lane, 0);
#pragma unroll
        for (int j = 0; j < kRadixKeysPerThread; ++j)
            key[j] = kFromFloat ? __float_as_uint(a.s[i0 + j * kWave]) : a.in[i0 + j * kWave];
    } else {
#pragma unroll
        for (int j = 0; j < kRadixKeysPerThread; ++j) {
            const int64_t i = key_index(base, wave, lane, j);
            const int64_t ic = i < a.n ? i : a.n - 1;
            key[j] = kFromFloat ? __float_as_uint(a.s[ic]) : a.in[ic];
        }
    }
    if (kFromFloat) {
#pragma unroll
        for (int j = 0; j < kRadixKeysPerThread; ++j)
            key[j] = float_to_key(__uint_as_float(key[j])) - a.key_min;
    }
}

}  // namespace

// Sub-histograms per work-group: four per wave (one per 16 lanes), rows
// padded to kHistStride words so one digit falls in a different LDS bank in
// each row.  A digit that many lanes share (the top digit of narrow-range
// scores, a tied cluster) then serialises over at most 16 lanes, and the
// round's most common digit (the first lane's) is counted by one add.
constexpr int kSubHists = kRadixWaves * 4;
constexpr int kHistStride = kRadixBins + 1;

template <bool kFromFloat>
__global__ __launch_bounds__(kRadixThreads) void radix_upsweep(PassArgs a)
{
    __shared__ uint32_t hist[kSubHists * kHistStride];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    for (int i = tid; i < kSubHists * kHistStride; i += kRadixThreads)
        hist[i] = 0;
    const int64_t base = (int64_t)blockIdx.x * kRadixTile;
    uint32_t key[kRadixKeysPerThread];
    load_keys<kFromFloat>(a, base, wave, lane, key);
    __syncthreads();  // sub-histograms cleared
    uint32_t* h = hist + (wave * 4 + lane / 16) * kHistStride;
#pragma unroll
    for (int j = 0; j < kRadixKeysPerThread; ++j) {
        const bool valid = key_index(base, wave, lane, j) < a.n;
        const uint32_t d = (key[j] >> a.shift) & 0xFFu;
        // valid lanes come first in every round, so lane 0 is valid
        // whenever any lane is
        const uint32_t d0 = __builtin_amdgcn_readfirstlane(d);
        const uint64_t same = __ballot(valid && d == d0);
        if (lane == 0 && same != 0)
            atomicAdd(&hist[wave * 4 * kHistStride + d0], (uint32_t)__popcll(same));
        if (valid && d != d0)
            atomicAdd(&h[d], 1u);
    }
    __syncthreads();
    uint32_t c = 0;
#pragma unroll
    for (int q = 0; q < kSubHists; ++q)
        c += hist[q * kHistStride + tid];
    a.hist[(size_t)blockIdx.x * kRadixBins + tid] = c;
}

// One work-group per chunk of tiles: per digit (one per thread), the sum
// of the chunk's rows.
__global__ __launch_bounds__(kRadixBins) void radix_chunk_sum(PassArgs a)
{
    const int d = threadIdx.x;
    const int t0 = blockIdx.x * a.chunk;
    const int t1 = t0 + a.chunk < a.g ? t0 + a.chunk : a.g;
    uint32_t s = 0;
#pragma unroll 8
    for (int t = t0; t < t1; ++t)
        s += a.hist[(size_t)t * kRadixBins + d];
    a.csum[(size_t)blockIdx.x * kRadixBins + d] = s;
}

// One work-group per chunk of tiles: per digit, the totals over all chunks
// (an exclusive scan of them over the digits gives the digit bases) and
// over the chunks before this one; then the chunk's rows become exclusive
// global offsets, tile by tile.
__global__ __launch_bounds__(kRadixBins) void radix_chunk_scan(PassArgs a)
{
    constexpr int kW = kRadixBins / kWave;
    __shared__ uint32_t wsum[kW];
    const int d = threadIdx.x;
    const int lane = d & (kWave - 1);
    const int wave = d / kWave;
    const int c = blockIdx.x;
    uint32_t tot = 0, pre = 0;
#pragma unroll 8
    for (int cc = 0; cc < a.chunks; ++cc) {
        const uint32_t v = a.csum[(size_t)cc * kRadixBins + d];
        tot += v;
        pre += cc < c ? v : 0u;
    }
    uint32_t incl = tot;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t v = __shfl_up(incl, o, kWave);
        if (lane >= o)
            incl += v;
    }
    if (lane == kWave - 1)
        wsum[wave] = incl;
    __syncthreads();
    uint32_t run = incl - tot + pre;  // digit base plus the earlier chunks
    for (int w = 0; w < wave; ++w)
        run += wsum[w];
    const int t0 = c * a.chunk;
    const int t1 = t0 + a.chunk < a.g ? t0 + a.chunk : a.g;
#pragma unroll 8
    for (int t = t0; t < t1; ++t) {
        const uint32_t v = a.hist[(size_t)t * kRadixBins + d];
        a.hist[(size_t)t * kRadixBins + d] = run;
        run += v;
    }
}

// The tile's keys are ranked stably into LDS in destination order (each
// digit's run in index order), then written out run by run, so the global
// stores go to consecutive addresses instead of 256 scattered buckets.  A
// digit's count in this tile is the step from its offset to the next
// tile's (or, for the last tile, to the next digit's base).
template <bool kFromFloat>
__global__ __launch_bounds__(kRadixThreads) void radix_downsweep(PassArgs a)
{
    __shared__ uint32_t goff[kRadixBins];
    __shared__ uint32_t lstart[kRadixBins];
    __shared__ uint32_t wrun[kRadixWaves][kRadixBins];  // a wave's running counts, then its prefix
    __shared__ uint32_t stage[kRadixTile];
    __shared__ uint32_t wsum[kRadixWaves];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int t = blockIdx.x;
    static_assert(kRadixThreads == kRadixBins, "one thread per digit");
    const int64_t base = (int64_t)t * kRadixTile;
    uint32_t key[kRadixKeysPerThread];
    load_keys<kFromFloat>(a, base, wave, lane, key);
    {
        // this thread's digit: global offset and count in this tile
        const int d = tid;
        const uint32_t off = a.hist[(size_t)t * kRadixBins + d];
        uint32_t next;
        if (t + 1 < a.g)
            next = a.hist[(size_t)(t + 1) * kRadixBins + d];
        else if (d + 1 < kRadixBins)
            next = a.hist[d + 1];  // tile 0's offset of the next digit: its base
        else
            next = (uint32_t)a.n;
        const uint32_t cnt = next - off;
        goff[d] = off;
#pragma unroll
        for (int w = 0; w < kRadixWaves; ++w)
            wrun[w][d] = 0;
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
    // ranks within this wave's 2048 keys, in index order: the wave's LDS
    // row is read by every lane, then advanced by the lowest lane of each
    // digit; one wave's LDS accesses take effect in program order, so no
    // barrier is needed between rounds
    // two ranks (each below 2048) per register
    uint32_t rk[kRadixKeysPerThread / 2];
#pragma unroll
    for (int j = 0; j < kRadixKeysPerThread; ++j) {
        const bool valid = key_index(base, wave, lane, j) < a.n;
        const uint32_t d = (key[j] >> a.shift) & 0xFFu;
        const uint64_t peers = match_digit(d, valid);
        const uint32_t below = rank_in_mask(peers);
        const uint32_t before = wrun[wave][d];
        if (j & 1)
            rk[j / 2] |= (before + below) << 16;
        else
            rk[j / 2] = before + below;
        if (valid && below == 0)
            wrun[wave][d] = before + (uint32_t)__popcll(peers);
    }
    __syncthreads();
    {
        // each digit's counts over the waves become the waves' starts
        const int d = tid;
        uint32_t run = 0;
#pragma unroll
        for (int w = 0; w < kRadixWaves; ++w) {
            const uint32_t c = wrun[w][d];
            wrun[w][d] = run;
            run += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRadixKeysPerThread; ++j) {
        if (key_index(base, wave, lane, j) < a.n) {
            const uint32_t d = (key[j] >> a.shift) & 0xFFu;
            stage[lstart[d] + wrun[wave][d] + ((rk[j / 2] >> (16 * (j & 1))) & 0xFFFFu)] = key[j];
        }
    }
    __syncthreads();
    const int64_t left = a.n - base;
    const int cnt = left < (int64_t)kRadixTile ? (int)left : kRadixTile;
    for (int j = tid; j < cnt; j += kRadixThreads) {
        const uint32_t k = stage[j];
        const uint32_t d = (k >> a.shift) & 0xFFu;
        a.out[goff[d] + (uint32_t)j - lstart[d]] = k;
    }
}

hipError_t launch_radix_sort(const RadixArgs& ra, hipStream_t stream)
{
    PassArgs a;
    a.s = ra.s;
    a.n = ra.n;
    a.g = ra.g_radix;
    a.chunk = radix_chunk_tiles(ra.g_radix);
    a.chunks = (ra.g_radix + a.chunk - 1) / a.chunk;  // <= kRadixMaxChunks
    a.hist = ra.hist;
    a.csum = ra.hist + (size_t)ra.g_radix * kRadixBins;
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
        STK_LAUNCH(kKRadixScan, stream, radix_chunk_sum, dim3(a.chunks), dim3(kRadixBins), 0, stream, a);
        STK_LAUNCH(kKRadixScan, stream, radix_chunk_scan, dim3(a.chunks), dim3(kRadixBins), 0, stream, a);
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
