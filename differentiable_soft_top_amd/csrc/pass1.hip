// pass1.hip -- the streaming and filtering pass of the bracketed solver.
//
// gist.science summary of Fast LapSum, section 2.2, "Probabilistic
// Bracketing" step 2: the whole score vector is streamed once; scores
// outside [a_L, a_R) are folded into tail sums, and only the middle band is
// kept.  Here, for every score s:
//   s <  a_L : nL += 1, SL += e^{(s - a_L)/alpha}      (exponent <= 0)
//   s >= a_R : nR += 1, SR += e^{-(s - a_R)/alpha}     (exponent <= 0)
//   else     : s is appended to the band.
// Both tails then enter the solve as two virtual nodes: for any b in
// [a_L, a_R] the left tail contributes SL e^{(a_L - b)/alpha} / 2 to M(b) and
// the right tail nR - SR e^{-(a_R - b)/alpha} / 2.
//
// Design for gfx950: the score vector is cut into tiles of 4096 scores
// (sixteen per lane: four 16-byte loads) taken in grid-stride order, so the
// resident work-groups sweep the vector together; two tiles' loads are issued
// at once and the first is classified while the second is in flight.  A tail score contributes
// 2^y with y = -|s - a|/alpha*log2e; below y = -50 the term is under 2^-50
// and is dropped (all dropped terms together stay below n * 2^-50 < 2e-6, far
// under the mass tolerance).  So a score is either "far" (s < t_L or
// s >= t_R: only counted, two fp32 compares and two carry adds) or inside the
// window [t_L, t_R), which holds the near tails and the band.  Window scores
// are compacted per wave into an LDS list (mask ranks, one store), and the
// wave then walks that list 64 at a time: near tail scores get the fp64
// exponential with every lane busy, band scores are appended with one LDS
// reservation per wave into a work-group stage, flushed with one global
// reservation per work-group (past the stage, in chunks of the global band;
// once a chunk ends past the buffer, the band has overflowed and the group
// only counts its band scores).  A NaN compares false both ways, so it lands in
// the window list and is flagged there; +-inf is caught by max |s|.  Counts
// are exact; sums are fp64; per-group partials are folded in fixed order by
// the consumer.
#include "stk_common.hpp"
#include "stk_layout.hpp"
#include "stk_prof.hpp"
#include "stk_reduce.hpp"

namespace stk {

namespace {

constexpr int kVals = 16;                       // scores per lane per tile
static_assert(kPass1Threads * kVals == kPass1TileScores, "tile size shared with the host");
constexpr int kTileQ = kPass1Threads * kVals / 4;  // float4 per tile
constexpr int kWin = kWave * kVals;             // window list per wave (worst case)
constexpr int kWaves1 = kPass1Threads / kWave;
constexpr double kTailCut = 50.0;               // tail terms below 2^-50 are dropped
constexpr int kP1Stage = 2048;                  // band scores staged per work-group
// A wave whose band scores overflow the stage takes the global band in
// chunks of kP1Chunk slots (one global reservation per chunk, not per
// batch); at the end the full stage fills every wave's unused chunk tail, so
// the band has no holes and its count stays exact.
constexpr int kP1Chunk = 512;
static_assert(kPass1Threads / kWave * kP1Chunk <= kP1Stage, "the stage covers every chunk tail");

struct Ctx1 {
    float aL, aR, tL, tR;
    double daL, daR, c;
    bool open;                                  // a bracket end is infinite: track the band range
    float* band;
    int64_t cap;
    unsigned long long* nB;
    float* stage;                               // LDS [kP1Stage]
    uint32_t* stage_count;                      // LDS reservation counter
    volatile uint32_t* full;                    // LDS: the group saw the band buffer full
    uint32_t* over;                             // LDS: band scores only counted since then
    float* win;                                 // this wave's LDS window list [kWin]
};

struct Acc1 {
    double SL, SR;
    uint32_t nL, nR;                            // per-lane counts of near tail scores
    uint32_t farL, farR;                        // wave-wide counts of far tail scores
    float bmin, bmax;
    float amax;                                 // max |s| (+-inf shows here)
    uint32_t nan;                               // a NaN reached the window list
    unsigned long long chunk_next;              // wave-uniform: next free slot of this wave's chunk
    uint32_t chunk_left;                        // wave-uniform: slots left in it
};

// Walk this wave's window list: near tail scores into the fp64 sums, band
// scores into the stage (or the global band past the stage).
__device__ __forceinline__ void drain_window(uint32_t cnt, const Ctx1& x, Acc1& acc)
{
    const int lane = lane_id();
    __builtin_amdgcn_wave_barrier();
    for (uint32_t base = 0; base < cnt; base += kWave) {
        const uint32_t j = base + (uint32_t)lane;
        const bool ok = j < cnt;
        const float s = ok ? x.win[j] : 0.f;
        const bool left = ok && s < x.aL;
        const bool right = ok && s >= x.aR;
        const bool nan = ok && s != s;
        const bool band = ok && !left && !right && !nan;
        acc.nL += left ? 1u : 0u;
        acc.nR += right ? 1u : 0u;
        acc.nan |= nan ? 1u : 0u;
        if (left || right) {
            const double d = left ? (double)s - x.daL : x.daR - (double)s;
            const double e = exp2_nonpos(d * x.c);
            if (left)
                acc.SL += e;
            else
                acc.SR += e;
        }
        const uint64_t mb = __builtin_amdgcn_ballot_w64(band);
        if (mb == 0)
            continue;
        const uint32_t total = (uint32_t)__popcll(mb);
        if (*x.full != 0u) {
            // the band has overflowed its buffer: only count (a reservation
            // per 512 band scores from here on would serialise on the
            // global counter)
            if (lane == 0)
                atomicAdd(x.over, total);
            if (band && x.open) {
                acc.bmin = fminf(acc.bmin, s);
                acc.bmax = fmaxf(acc.bmax, s);
            }
            continue;
        }
        uint32_t sbase = 0;
        if (lane == 0)
            sbase = atomicAdd(x.stage_count, total);
        sbase = __shfl(sbase, 0, kWave);
        // reservations past the LDS stage go to this wave's chunk of the
        // global band (a new chunk when it runs out; n_over <= 64 < kP1Chunk)
        const uint32_t first_over = sbase > (uint32_t)kP1Stage ? sbase : (uint32_t)kP1Stage;
        const uint32_t end = sbase + total;
        const uint32_t n_over = end > first_over ? end - first_over : 0u;
        uint32_t take = 0;
        unsigned long long g0 = 0, g1 = 0;
        if (n_over) {
            take = n_over < acc.chunk_left ? n_over : acc.chunk_left;
            g0 = acc.chunk_next;
            acc.chunk_next += take;
            acc.chunk_left -= take;
            if (take < n_over) {
                unsigned long long nb = 0;
                if (lane == 0)
                    nb = atomicAdd(x.nB, (unsigned long long)kP1Chunk);
                nb = __shfl(nb, 0, kWave);
                g1 = nb;
                acc.chunk_next = nb + (n_over - take);
                acc.chunk_left = (uint32_t)kP1Chunk - (n_over - take);
                // a chunk that ends past the buffer: the count now exceeds
                // the capacity, so the band overflows whatever follows
                if (lane == 0 && nb + (unsigned long long)kP1Chunk > (unsigned long long)x.cap)
                    *x.full = 1u;
            }
        }
        if (band) {
            const uint32_t pos = sbase + rank_in_mask(mb);
            if (x.open) {
                acc.bmin = fminf(acc.bmin, s);
                acc.bmax = fmaxf(acc.bmax, s);
            }
            if (pos < (uint32_t)kP1Stage) {
                x.stage[pos] = s;
            } else {
                const uint32_t o = pos - first_over;  // rank among this batch's overflow
                const uint64_t g = o < take ? (uint64_t)g0 + o : (uint64_t)g1 + (o - take);
                if (g < (uint64_t)x.cap)
                    x.band[g] = s;
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
}

// Classify kVals scores of this lane (kAll: all valid, else bit i of
// `valid`).  Far scores are counted; window scores are compacted into the
// wave's list, which is then drained.  Called by every lane of the wave.
// The far counts are wave-wide (scalar popcounts of the compare masks):
// far-left directly, far-right as what is neither far-left nor in the
// window.
template <bool kAll>
__device__ __forceinline__ void classify(const float (&v)[kVals], uint32_t valid, const Ctx1& x, Acc1& acc)
{
    uint32_t cnt = 0;   // wave-uniform fill of the window list
    uint32_t lo_n = 0;  // wave-uniform far-left count
    uint32_t ok_n = 0;  // wave-uniform count of valid scores
    const uint64_t live = __builtin_amdgcn_ballot_w64(true);
#pragma unroll
    for (int i = 0; i < kVals; ++i) {
        const bool ok = kAll || ((valid >> i) & 1u);
        const float s = v[i];
        const bool lo = s < x.tL;
        const bool hi = s >= x.tR;
        acc.amax = fmaxf(acc.amax, ok ? fabsf(s) : 0.f);
        // window mask from the ballots of the two compares (stays scalar)
        const uint64_t mlo = __builtin_amdgcn_ballot_w64(lo);
        uint64_t m = ~(mlo | __builtin_amdgcn_ballot_w64(hi)) & live;
        uint64_t mok = live;
        if (!kAll) {
            mok = __builtin_amdgcn_ballot_w64(ok);
            m &= mok;
        }
        lo_n += (uint32_t)__popcll(mlo & mok);
        ok_n += (uint32_t)__popcll(mok);
        if (ok && !lo && !hi)  // this lane's bit of m
            x.win[cnt + rank_in_mask(m)] = s;
        cnt += (uint32_t)__popcll(m);
    }
    acc.farL += lo_n;
    acc.farR += ok_n - lo_n - cnt;
    drain_window(cnt, x, acc);
}

template <int kU>
__device__ __forceinline__ void classify_q(const float4 (&f)[kU], const Ctx1& x, Acc1& acc)
{
    float v[kVals];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        v[4 * u + 0] = f[u].x;
        v[4 * u + 1] = f[u].y;
        v[4 * u + 2] = f[u].z;
        v[4 * u + 3] = f[u].w;
    }
    classify<true>(v, 0xFFFFu, x, acc);
}

template <int kU>
__device__ __forceinline__ void load_tile(const float4* __restrict__ s4, int64_t t, float4 (&f)[kU])
{
#pragma unroll
    for (int u = 0; u < kU; ++u)
        f[u] = s4[t * (kU * kPass1Threads) + u * kPass1Threads + threadIdx.x];
}

}  // namespace

template <bool kVec>
__global__ __launch_bounds__(kPass1Threads) void pass1_kernel(Pass1Args a)
{
    __shared__ float stage_buf[kP1Stage];
    __shared__ float win_buf[kWaves1][kWin];
    __shared__ uint32_t stage_count;
    __shared__ uint32_t band_full, band_over;
    __shared__ unsigned long long stage_base;
    __shared__ unsigned long long tail_at[kWaves1];
    __shared__ uint32_t tail_n[kWaves1];
    __shared__ double red_d[2][kWaves1];
    __shared__ uint32_t red_u[3][kWaves1];
    __shared__ float red_f[3][kWaves1];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    Status* st = a.st;

    if (tid == 0) {
        stage_count = 0;
        band_full = a.count_only != 0 ? 1u : 0u;  // counting only from the start
        band_over = 0;
    }
    __syncthreads();

    Ctx1 x;
    x.aL = st->aL;
    x.aR = st->aR;
    x.daL = x.aL;
    x.daR = x.aR;
    x.c = a.log2e_over_alpha;
    // window ends in fp32, rounded outward so no term >= 2^-50 is dropped
    const double cut = kTailCut / x.c;
    x.tL = (float)(x.daL - cut);
    if ((double)x.tL > x.daL - cut)
        x.tL = nextafterf(x.tL, -INFINITY);
    x.tR = (float)(x.daR + cut);
    if ((double)x.tR < x.daR + cut)
        x.tR = nextafterf(x.tR, INFINITY);
    x.open = (x.aL == -INFINITY) || (x.aR == INFINITY);
    x.band = a.band;
    x.cap = a.cap;
    x.nB = reinterpret_cast<unsigned long long*>(&st->nB);
    x.stage = stage_buf;
    x.stage_count = &stage_count;
    x.full = &band_full;
    x.over = &band_over;
    x.win = win_buf[wave];

    Acc1 acc{0.0, 0.0, 0u, 0u, 0u, 0u, INFINITY, -INFINITY, 0.f, 0u, 0ull, 0u};
    const int64_t G = gridDim.x;
    int64_t rest = 0;  // first score not covered by whole tiles

    if (kVec) {
        const int64_t n4 = a.n >> 2;
        const int64_t T = n4 / kTileQ;
        const float4* s4 = reinterpret_cast<const float4*>(a.s);
        constexpr int kU = kVals / 4;
        // each step issues the loads of two tiles (eight 16-byte loads per
        // lane) and classifies the first while the second is in flight
        int64_t t = blockIdx.x;
        for (; t + G < T; t += 2 * G) {
            float4 fa[kU], fb[kU];
            load_tile<kU>(s4, t, fa);
            load_tile<kU>(s4, t + G, fb);
            classify_q<kU>(fa, x, acc);
            classify_q<kU>(fb, x, acc);
        }
        if (t < T) {
            float4 fa[kU];
            load_tile<kU>(s4, t, fa);
            classify_q<kU>(fa, x, acc);
        }
        rest = T * (int64_t)kTileQ * 4;
        // the ragged end (a partial tile and the last n mod 4 scores) goes to
        // the work-group whose next tile it would be
        if ((T - (int64_t)blockIdx.x) % G != 0)
            rest = a.n;
    } else {
        // unaligned scores: plain grid-stride over scalar loads
        for (int64_t i0 = (int64_t)blockIdx.x * (kPass1Threads * kVals); i0 < a.n;
             i0 += G * (kPass1Threads * kVals)) {
            float v[kVals];
            uint32_t valid = 0;
#pragma unroll
            for (int k = 0; k < kVals; ++k) {
                const int64_t i = i0 + (int64_t)k * kPass1Threads + tid;
                v[k] = i < a.n ? a.s[i] : 0.f;
                valid |= (i < a.n ? 1u : 0u) << k;
            }
            classify<false>(v, valid, x, acc);
        }
        rest = a.n;
    }
    for (int64_t i0 = rest; i0 < a.n; i0 += kPass1Threads * kVals) {
        float v[kVals];
        uint32_t valid = 0;
#pragma unroll
        for (int k = 0; k < kVals; ++k) {
            const int64_t i = i0 + (int64_t)k * kPass1Threads + tid;
            v[k] = i < a.n ? a.s[i] : 0.f;
            valid |= (i < a.n ? 1u : 0u) << k;
        }
        classify<false>(v, valid, x, acc);
    }

    // flush the LDS stage: its first entries fill the waves' unused chunk
    // tails (a chunk exists only once the stage is full, and the tails add up
    // to at most the stage), the rest takes one global reservation
    if (lane == 0) {
        tail_at[wave] = acc.chunk_next;
        tail_n[wave] = acc.chunk_left;
    }
    __syncthreads();
    uint32_t tails = 0;
    for (int w = 0; w < kWaves1; ++w)
        tails += tail_n[w];
    const uint32_t staged = stage_count < (uint32_t)kP1Stage ? stage_count : (uint32_t)kP1Stage;
    if (tid == 0) {
        stage_base = staged > tails ? atomicAdd(x.nB, (unsigned long long)(staged - tails)) : 0ull;
        if (band_over != 0u)  // the counted-only band scores keep the band count exact
            atomicAdd(x.nB, (unsigned long long)band_over);
    }
    __syncthreads();
    for (uint32_t i = tid; i < staged; i += kPass1Threads) {
        uint64_t g;
        if (i < tails) {
            uint32_t r = i;
            int w = 0;
            while (r >= tail_n[w]) {
                r -= tail_n[w];
                ++w;
            }
            g = tail_at[w] + r;
        } else {
            g = (uint64_t)stage_base + (i - tails);
        }
        if (g < (uint64_t)a.cap)
            a.band[g] = stage_buf[i];
    }

    // work-group reduction into this group's partial; the consumer (segment
    // solve) folds the partials in fixed order.  No ticket: an agent-scope
    // fence per work-group would write back the whole L2 each time.
    const double SL = wave_sum(acc.SL);
    const double SR = wave_sum(acc.SR);
    // far counts are the same in every lane of a wave: counted once
    const uint32_t nL = wave_sum_u32(acc.nL) + acc.farL;
    const uint32_t nR = wave_sum_u32(acc.nR) + acc.farR;
    uint32_t nf = (acc.nan != 0u || !(acc.amax < INFINITY)) ? 1u : 0u;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        nf |= __shfl_xor(nf, off, kWave);
    const float bmin = wave_min(acc.bmin), bmax = wave_max(acc.bmax);
    if (lane == 0) {
        red_d[0][wave] = SL;
        red_d[1][wave] = SR;
        red_u[0][wave] = nL;
        red_u[1][wave] = nR;
        red_u[2][wave] = nf;
        red_f[0][wave] = bmin;
        red_f[1][wave] = bmax;
    }
    __syncthreads();
    if (tid == 0) {
        Pass1Partial p;
        p.SL = 0.0;
        p.SR = 0.0;
        p.nL = 0;
        p.nR = 0;
        p.nonfinite = 0;
        p.bmin = INFINITY;
        p.bmax = -INFINITY;
        p.smin = INFINITY;
        p.smax = -INFINITY;
        for (int w = 0; w < kWaves1; ++w) {
            p.SL += red_d[0][w];
            p.SR += red_d[1][w];
            p.nL += red_u[0][w];
            p.nR += red_u[1][w];
            p.nonfinite |= red_u[2][w];
            p.bmin = fminf(p.bmin, red_f[0][w]);
            p.bmax = fmaxf(p.bmax, red_f[1][w]);
        }
        a.partials[blockIdx.x] = p;
    }
}

// ---------------------------------------------------------------------------
// Score range and finiteness for the full-sort route (the radix sort only
// sorts the key bits that vary between the smallest and largest score).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kStreamThreads) void range_kernel(const float* __restrict__ s, int64_t n,
                                                               Pass1Partial* partials, int blocks)
{
    __shared__ float red[3][kStreamThreads / kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int64_t i0 = (n * blockIdx.x) / blocks;
    const int64_t i1 = (n * (blockIdx.x + 1)) / blocks;
    float mn = INFINITY, mx = -INFINITY, nf = 0.f;
    // eight loads in flight per lane; past i1 a load repeats the range's
    // first score (no branch around a load; a repeat changes no extreme)
    constexpr int kU = 8;
    for (int64_t i = i0 + tid; i < i1; i += kU * kStreamThreads) {
        float v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t j = i + (int64_t)u * kStreamThreads;
            v[u] = s[j < i1 ? j : i0];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            mn = fminf(mn, v[u]);
            mx = fmaxf(mx, v[u]);
            nf = fmaf(v[u], 0.f, nf);
        }
    }
    uint32_t bad = (nf != 0.f || nf != nf) ? 1u : 0u;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        bad |= __shfl_xor(bad, off, kWave);
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
        red[0][wave] = mn;
        red[1][wave] = mx;
        red[2][wave] = bad ? 1.f : 0.f;
    }
    __syncthreads();
    if (tid == 0) {
        Pass1Partial p;
        p.SL = 0.0;
        p.SR = 0.0;
        p.nL = 0;
        p.nR = 0;
        p.bmin = INFINITY;
        p.bmax = -INFINITY;
        p.smin = INFINITY;
        p.smax = -INFINITY;
        p.nonfinite = 0;
        for (int w = 0; w < kStreamThreads / kWave; ++w) {
            p.smin = fminf(p.smin, red[0][w]);
            p.smax = fmaxf(p.smax, red[1][w]);
            p.nonfinite |= red[2][w] != 0.f ? 1u : 0u;
        }
        partials[blockIdx.x] = p;
    }
}

hipError_t launch_range(const float* s, int64_t n, Pass1Partial* partials, int blocks, hipStream_t stream)
{
    STK_LAUNCH(kKPass1, stream, range_kernel, dim3(blocks), dim3(kStreamThreads), 0, stream, s, n, partials, blocks);
    return hipGetLastError();
}

__global__ __launch_bounds__(kStreamThreads) void pass1_finalize_kernel(const Pass1Partial* partials, int blocks,
                                                                        Status* st)
{
    reduce_pass1(partials, blocks, st);
}

hipError_t launch_pass1_finalize(const Pass1Partial* partials, int blocks, Status* st, hipStream_t stream)
{
    STK_LAUNCH(kKReset, stream, pass1_finalize_kernel, dim3(1), dim3(kStreamThreads), 0, stream, partials, blocks, st);
    return hipGetLastError();
}

hipError_t launch_pass1(const Pass1Args& a, hipStream_t stream)
{
    const bool vec = (reinterpret_cast<uintptr_t>(a.s) & 15u) == 0;
    if (vec)
        STK_LAUNCH(kKPass1, stream, pass1_kernel<true>, dim3(a.blocks), dim3(kPass1Threads), 0, stream, a);
    else
        STK_LAUNCH(kKPass1, stream, pass1_kernel<false>, dim3(a.blocks), dim3(kPass1Threads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace stk
