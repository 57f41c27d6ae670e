// dftopk.hip -- the DFTopK comparator's threshold: the midpoint of the k-th
// and (k+1)-th largest scores.
//
// mlsanity.com page "Differentiable Fast Top-K Selection for Large-Scale
// Recommendation" (abstract): DFTopK relaxes the budget constraint so that
// the threshold needs no sort.  gist.science summary of Fast LapSum, section
// 2.3 "Relation to DFTopK": it fixes b at the midpoint of the k-th and
// (k+1)-th order statistics, which is LapSum's zero-temperature limit; at a
// finite temperature the selected mass sum_i F((s_i - b)/alpha) then drifts
// away from k, where LapSum keeps it exact.  The emission afterwards is
// LapSum's own (emit_vjp.hip), at this b.
//
// gfx950 design: an exact most-significant-digit radix selection of the two
// order statistics over the order-preserving u32 keys of the scores, three
// streaming passes of 11, 11 and 10 bits, with no host synchronisation:
//   pass P (dft_hist_kernel<P>) -- every work-group first works out, from
//     the previous pass's totals, which digit prefix each target continues
//     (its own copy of a small scan; work-group 0 records it), then streams
//     its share of the scores and counts, for each target, the next digit of
//     the keys that carry the target's prefix, in an LDS histogram (one
//     histogram while the two targets' prefixes agree).  A wave merges the
//     lanes that share its first lane's digit into one add, so a tied
//     cluster costs no atomic contention.  Each work-group writes its
//     histograms as one row.
//   fold (dft_fold_kernel) -- the rows are summed column by column, in
//     chunks of rows spread over many work-groups.
//   finalize (dft_finalize_kernel) -- the last digit completes both keys;
//     b = (x_(k) + x_(k+1)) / 2 in fp64.
// A NaN score makes b NaN (and every p NaN); infinities are ordered like
// any other value.  Ranks are exact and ties need no care: the selection
// returns the value at each rank.
#include "stk_common.hpp"
#include "stk_layout.hpp"

namespace stk {

namespace {

constexpr int kDT = kDftThreads;
constexpr int kDW = kDT / kWave;
constexpr int kDQ = 8;                  // float4 per lane per tile
constexpr int kDTile = kDT * kDQ * 4;   // scores per tile

__device__ __forceinline__ int dft_shift(int P) { return P == 0 ? 21 : (P == 1 ? 10 : 0); }
__device__ __forceinline__ int dft_width(int P) { return P == 2 ? 10 : 11; }

// The state before pass P + 1 from the state before pass P and pass P's
// totals, for both targets: the digit whose count range holds the target's
// remaining rank extends its prefix, and the counts below it leave the rank.
// Every thread of the work-group calls it; the result is in *out.
__device__ void dft_select(const DftState& in, const uint32_t* totals, int P, DftState* out, uint32_t* lds_sum)
{
    const int bins = 1 << dft_width(P);
    const int per = bins / kDT;  // bins per thread (8 or 4)
    const int tid = threadIdx.x;
    for (int t = 0; t < 2; ++t) {
        const uint32_t* cnt = totals + t * kDftBins;
        uint32_t mine = 0u;
        for (int j = 0; j < per; ++j)
            mine += cnt[tid * per + j];
        // exclusive scan of the per-thread sums (inclusive wave scan, then
        // the wave totals through LDS)
        uint32_t inc = mine;
        const int lane = lane_id();
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const uint32_t o = __shfl_up(inc, off, kWave);
            if (lane >= off)
                inc += o;
        }
        if (lane == kWave - 1)
            lds_sum[tid / kWave] = inc;
        __syncthreads();
        uint32_t before = inc - mine;
        for (int w = 0; w < tid / kWave; ++w)
            before += lds_sum[w];
        const uint32_t r = in.rank[t];
        if (r >= before && r < before + mine) {
            uint32_t cum = before;
            for (int j = 0; j < per; ++j) {
                const uint32_t c = cnt[tid * per + j];
                if (r < cum + c) {
                    out->prefix[t] = (in.prefix[t] << dft_width(P)) | (uint32_t)(tid * per + j);
                    out->rank[t] = r - cum;
                    break;
                }
                cum += c;
            }
        }
        __syncthreads();  // lds_sum reused by the next target
    }
}

// One slot's digit counted for the lanes that `match`, in one LDS atomic
// instruction: the lanes that share the first matching lane's digit are
// merged into that lane's add (a tied cluster or a narrow range costs one
// add, not a 64-way conflict), every other matching lane adds one.  Merging
// further digits measured slower on spread data (more instructions per
// slot, while the spread adds rarely collide).
__device__ __forceinline__ void agg_count(uint32_t* h, bool match, uint32_t d)
{
    const uint64_t active = __ballot(match);
    if (active == 0ull)
        return;
    const int leader = (int)__builtin_ctzll(active);
    const uint32_t dl = (uint32_t)__builtin_amdgcn_readlane((int)d, leader);
    const uint64_t same = __ballot(match && d == dl);
    const bool lead = lane_id() == leader;
    if (match && (lead || d != dl))
        atomicAdd(&h[d], lead ? (uint32_t)__popcll(same) : 1u);
}

template <int P>
__device__ __forceinline__ void dft_count(float v, const DftState& S, uint32_t (*h)[kDftBins], uint32_t* nan_cnt)
{
    constexpr int kShift = P == 0 ? 21 : (P == 1 ? 10 : 0);
    constexpr uint32_t kMask = P == 2 ? 1023u : 2047u;
    const uint32_t key = float_to_key(v);
    const uint32_t d = (key >> kShift) & kMask;
    if (P == 0) {
        agg_count(h[0], true, d);
        const uint64_t nanm = __ballot(v != v);
        if (nanm != 0ull && lane_id() == 0)
            atomicAdd(nan_cnt, (uint32_t)__popcll(nanm));
    } else {
        constexpr int kAbove = P == 1 ? 21 : 10;
        agg_count(h[0], (key >> kAbove) == S.prefix[0], d);
        if (S.prefix[1] != S.prefix[0])  // both targets share one histogram when their prefixes agree
            agg_count(h[1], (key >> kAbove) == S.prefix[1], d);
    }
}

template <int P>
__global__ __launch_bounds__(kDT) void dft_hist_kernel(DftArgs a)
{
    __shared__ uint32_t h[2][kDftBins];
    __shared__ uint32_t nan_cnt;
    __shared__ uint32_t lds_sum[kDW];
    __shared__ DftState S;
    const int tid = threadIdx.x;
    for (int i = tid; i < 2 * kDftBins; i += kDT)
        (&h[0][0])[i] = 0u;
    if (tid == 0) {
        nan_cnt = 0u;
        if (P == 0) {
            // ascending 0-based ranks: the (k+1)-th largest, then the k-th
            S.prefix[0] = S.prefix[1] = 0u;
            S.rank[0] = (uint32_t)(a.n - a.k - 1);
            S.rank[1] = (uint32_t)(a.n - a.k);
        }
    }
    if (P > 0) {
        __syncthreads();
        dft_select(a.state[P - 1], a.totals + (size_t)(P - 1) * kDftRowWords, P - 1, &S, lds_sum);
    }
    __syncthreads();
    if (blockIdx.x == 0) {
        if (tid == 0)
            a.state[P] = S;  // the state before this pass, for the next pass and the finalize
        // this pass's totals, folded by the next kernel
        for (int i = tid; i < kDftRowWords; i += kDT)
            a.totals[(size_t)P * kDftRowWords + i] = 0u;
    }
    const DftState Sr = S;

    const int64_t G = gridDim.x;
    const bool vec = (reinterpret_cast<uintptr_t>(a.s) & 15u) == 0;
    int64_t done = 0;
    if (vec) {
        const int64_t T = a.n / kDTile;
        const float4* s4 = reinterpret_cast<const float4*>(a.s);
        for (int64_t t = blockIdx.x; t < T; t += G) {
            float4 f[kDQ];
#pragma unroll
            for (int u = 0; u < kDQ; ++u)
                f[u] = s4[t * (kDT * kDQ) + u * kDT + tid];
#pragma unroll
            for (int u = 0; u < kDQ; ++u) {
                dft_count<P>(f[u].x, Sr, h, &nan_cnt);
                dft_count<P>(f[u].y, Sr, h, &nan_cnt);
                dft_count<P>(f[u].z, Sr, h, &nan_cnt);
                dft_count<P>(f[u].w, Sr, h, &nan_cnt);
            }
        }
        done = T * kDTile;
    }
    // the ragged end (or an unaligned vector): one score per lane; every
    // lane of a wave takes the slot loop together (the ballots need it)
    const int64_t rest = a.n - done;
    const int64_t per_group = (rest + G - 1) / G;
    const int64_t i0 = done + (int64_t)blockIdx.x * per_group;
    const int64_t i1 = i0 + per_group < a.n ? i0 + per_group : a.n;
    for (int64_t base = i0; base < i1; base += kDT) {
        const int64_t i = base + tid;
        const bool in = i < i1;
        const float v = in ? a.s[i] : 0.0f;
        const uint32_t key = float_to_key(v);
        if (P == 0) {
            agg_count(h[0], in, (key >> 21) & 2047u);
            const uint64_t nanm = __ballot(in && v != v);
            if (nanm != 0ull && lane_id() == 0)
                atomicAdd(&nan_cnt, (uint32_t)__popcll(nanm));
        } else {
            const int above = P == 1 ? 21 : 10;
            const uint32_t d = (key >> dft_shift(P)) & (P == 2 ? 1023u : 2047u);
            agg_count(h[0], in && (key >> above) == Sr.prefix[0], d);
            if (Sr.prefix[1] != Sr.prefix[0])
                agg_count(h[1], in && (key >> above) == Sr.prefix[1], d);
        }
    }
    __syncthreads();
    uint32_t* row = a.rows + (size_t)blockIdx.x * kDftRowWords;
    for (int i = tid; i < kDftBins; i += kDT) {
        row[i] = h[0][i];
        // pass 0, and a later pass whose two prefixes agree: one histogram
        row[kDftBins + i] = P == 0 || Sr.prefix[1] == Sr.prefix[0] ? h[0][i] : h[1][i];
    }
    if (tid == 0)
        row[2 * kDftBins] = nan_cnt;
}

// totals[P][col] = sum over the work-group rows of rows[g][col].  A
// work-group takes 64 columns (one per lane) of kFoldRows rows; its waves
// take every kDW-th row, with all their loads in flight at once, and meet
// in LDS; one atomic per non-zero column folds the chunk into the totals,
// which pass P's work-group 0 cleared.
constexpr int kFoldRows = 8 * kDW;
static_assert(kDftRowWords % kWave == 0, "fold columns come in whole waves");

__global__ __launch_bounds__(kDT) void dft_fold_kernel(DftArgs a, int P)
{
    __shared__ uint32_t part[kDW][kWave];
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int col = blockIdx.x * kWave + lane;
    const int g0 = blockIdx.y * kFoldRows;
    const bool live = col <= 2 * kDftBins;  // the padding columns are never written
    uint32_t v[kFoldRows / kDW];
#pragma unroll
    for (int j = 0; j < kFoldRows / kDW; ++j) {
        const int g = g0 + j * kDW + wave;
        v[j] = live && g < a.groups ? a.rows[(size_t)g * kDftRowWords + col] : 0u;
    }
    uint32_t t = 0u;
#pragma unroll
    for (int j = 0; j < kFoldRows / kDW; ++j)
        t += v[j];
    part[wave][lane] = t;
    __syncthreads();
    if (wave == 0) {
        t = 0u;
#pragma unroll
        for (int w = 0; w < kDW; ++w)
            t += part[w][lane];
        if (t != 0u)
            atomicAdd(&a.totals[(size_t)P * kDftRowWords + col], t);
    }
}

__global__ __launch_bounds__(kDT) void dft_finalize_kernel(DftArgs a)
{
    __shared__ uint32_t lds_sum[kDW];
    __shared__ DftState S;
    dft_select(a.state[2], a.totals + 2 * (size_t)kDftRowWords, 2, &S, lds_sum);
    __syncthreads();
    if (threadIdx.x == 0) {
        Status* st = a.st;
        const bool nan = a.totals[2 * kDftBins] != 0u;  // pass 0's NaN count
        const float lo = key_to_float(S.prefix[0]);     // (k+1)-th largest
        const float hi = key_to_float(S.prefix[1]);     // k-th largest
        const double b = nan ? (double)NAN : 0.5 * ((double)hi + (double)lo);
        st->b = b;
        *a.out_b = b;
        st->solve_state = nan ? kSolveNonfinite : kSolveOk;
        st->nonfinite = nan ? 1u : 0u;
        st->emit_done = 0;
        st->seg_valid = 0;
        st->aL = lo;
        st->aR = hi;
    }
}

// After the emission (and its mass fold when asked): NaN input fills p with
// NaN, and the mass goes to the caller.
__global__ __launch_bounds__(kStreamThreads) void dft_tail_kernel(const Status* st, float* p, int64_t n,
                                                                   double* out_mass)
{
    const bool nan = st->solve_state == kSolveNonfinite;
    if (blockIdx.x == 0 && threadIdx.x == 0 && out_mass != nullptr)
        *out_mass = (!nan && st->emit_done) ? st->mass : (double)NAN;
    if (!nan)
        return;
    for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kStreamThreads)
        p[i] = NAN;
}

}  // namespace

hipError_t launch_dftopk_threshold(const DftArgs& a, hipStream_t stream)
{
    const dim3 block(kDT), gh(a.groups), gf(kDftRowWords / kWave, (a.groups + kFoldRows - 1) / kFoldRows);
    dft_hist_kernel<0><<<gh, block, 0, stream>>>(a);
    dft_fold_kernel<<<gf, block, 0, stream>>>(a, 0);
    dft_hist_kernel<1><<<gh, block, 0, stream>>>(a);
    dft_fold_kernel<<<gf, block, 0, stream>>>(a, 1);
    dft_hist_kernel<2><<<gh, block, 0, stream>>>(a);
    dft_fold_kernel<<<gf, block, 0, stream>>>(a, 2);
    dft_finalize_kernel<<<1, block, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_dftopk_tail(const Status* st, float* p, int64_t n, double* out_mass, int32_t blocks,
                              hipStream_t stream)
{
    dft_tail_kernel<<<blocks, kStreamThreads, 0, stream>>>(st, p, n, out_mass);
    return hipGetLastError();
}

}  // namespace stk
