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
        st->seg_valid = 0;
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
        publish_status(st, a.mirror, 0u);
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
    publish_status(st, a.mirror, 0u);
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
            // fp64 sums of fp32 d and exact g d products: where one d
            // dominates, g_i - G/D is small and needs G and D to far better
            // than fp32 rounding of the dominant term
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                acc_dg(dens(vs[u].x, b, c), vg[u].x, D, G_);
                acc_dg(dens(vs[u].y, b, c), vg[u].y, D, G_);
                acc_dg(dens(vs[u].z, b, c), vg[u].z, D, G_);
                acc_dg(dens(vs[u].w, b, c), vg[u].w, D, G_);
            }
        }
        for (int64_t i = ragged_start<kB>(a.n, T) + tid; i < a.n; i += kStreamThreads) {
            acc_dg(dens(a.s[i], b, c), a.g[i], D, G_);
        }
    } else {
        for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + tid; i < a.n; i += G * kStreamThreads) {
            acc_dg(dens(a.s[i], b, c), a.g[i], D, G_);
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
    const Ratio2 ratio = split_ratio(tot[0] > 0.0 ? tot[1] / tot[0] : 0.0);
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
                o.x = dens(vs[u].x, b, c) * inv_alpha * minus_ratio(vg[u].x, ratio);
                o.y = dens(vs[u].y, b, c) * inv_alpha * minus_ratio(vg[u].y, ratio);
                o.z = dens(vs[u].z, b, c) * inv_alpha * minus_ratio(vg[u].z, ratio);
                o.w = dens(vs[u].w, b, c) * inv_alpha * minus_ratio(vg[u].w, ratio);
                store4<kNT>(&o4[t * (kB * kStreamThreads) + u * kStreamThreads + tid], o);
            }
        }
        for (int64_t i = ragged_start<kB>(a.n, T) + tid; i < a.n; i += kStreamThreads)
            a.grad[i] = dens(a.s[i], b, c) * inv_alpha * minus_ratio(a.g[i], ratio);
    } else {
        for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + tid; i < a.n; i += G * kStreamThreads)
            a.grad[i] = dens(a.s[i], b, c) * inv_alpha * minus_ratio(a.g[i], ratio);
    }
}

// ---------------------------------------------------------------------------
// Saturated-score segments (from kSegMinN scores on, aligned vectors).  The
// emission, which knows b, records for each wave's 1024-score share of a
// large VJP tile the scores whose fp32 density d_i = dens(s_i) is at least
// kDensCut = 2^-40 (|s_i - b| < 27.7 alpha) and, when there are at most
// kSegCap, their d values and their places in the segment.  The VJP then
// reads those instead of the scores: its reduction takes d from the record
// and 0 elsewhere (dropping terms below 2^-40, which moves D and G by at most
// n 2^-40 and no gradient element by more than 2^-39 of the largest one) and
// stores the matching g values, compacted, in its workspace; its gradient
// kernel reads only the compacted (d, g, place) triples and writes +0 for the
// other scores.  If G is not finite (a non-finite g) the gradient kernel
// reads the scores throughout.
//
// A segment's place p of element i of lane l (the element at float4
// tile * 1024 + (i / 4) * 256 + wave * 64 + l, component i mod 4) is
// (i / 4) * 256 + l * 4 + (i mod 4): its offset in the wave's 1024-float LDS
// tile when each lane stores its four float4 at float4 offset u * 64 + l.  So
// the VJP moves whole float4 between registers and LDS and touches single
// floats only for the listed scores -- one LDS access per listed score
// instead of a ballot, a rank and a select per score.
// ---------------------------------------------------------------------------
namespace {

constexpr float kDensCut = 0x1p-40f;                  // densities the record keeps (at least)
constexpr int kSegV = 4 * kVjpBatchLarge;             // values per lane in a segment
constexpr int kSegPerTile = kStreamThreads / kWave;   // segments per large VJP tile
constexpr int kCntChunk = 8;                          // tiles whose counts are fetched at once
static_assert(kSegV == 16 && kSegScores == kSegV * kWave && (kSegCap & (kSegCap - 1)) == 0 && kSegCap >= 64,
              "segment record: 16 values per lane; power-of-two value regions");

__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }

constexpr int kSegSteps = kSegCap / kWave;

// The counts of this wave's segments of tiles tile(c), c < kCntChunk
// (tiles without a record, or past the vector, read as dense).
template <typename TileOf>
__device__ __forceinline__ void fetch_counts(const VjpArgs& a, TileOf tile_of, int64_t T, uint32_t (&cnt)[kCntChunk])
{
    const int wave = wave_index();
    const int64_t Ts = a.seg_tiles < T ? a.seg_tiles : T;
#pragma unroll
    for (int c = 0; c < kCntChunk; ++c) {
        const int64_t t = tile_of(c);
        const bool has = t >= 0 && t < Ts;
        cnt[c] = has ? a.seg.cnt[(has ? t : 0) * kSegPerTile + wave] : kSegDense;
    }
}

// The wave's four float4 per lane into / out of its LDS tile.
__device__ __forceinline__ void tile_store(float* tile, const float4 (&v)[kVjpBatchLarge])
{
    float4* t4 = reinterpret_cast<float4*>(tile);
#pragma unroll
    for (int u = 0; u < kVjpBatchLarge; ++u)
        t4[u * kWave + lane_id()] = v[u];
}

__device__ __forceinline__ void tile_load(const float* tile, float4 (&v)[kVjpBatchLarge])
{
    const float4* t4 = reinterpret_cast<const float4*>(tile);
#pragma unroll
    for (int u = 0; u < kVjpBatchLarge; ++u)
        v[u] = t4[u * kWave + lane_id()];
}

// A record entry: the listed score's fp32 density d (low word) and its
// place in the segment (high word), one 8-byte store and load.
__device__ __forceinline__ uint64_t seg_entry(float d, uint32_t place)
{
    return ((uint64_t)place << 32) | (uint64_t)__float_as_uint(d);
}
__device__ __forceinline__ float entry_d(uint64_t e) { return __uint_as_float((uint32_t)e); }
__device__ __forceinline__ uint32_t entry_place(uint64_t e) { return (uint32_t)(e >> 32) & (kSegScores - 1); }

// Whether every segment of a chunk has a record listing at most one value
// per lane (the common case away from b).
__device__ __forceinline__ bool chunk_is_light(const uint32_t (&cnt)[kCntChunk])
{
    bool ok = true;
#pragma unroll
    for (int c = 0; c < kCntChunk; ++c)
        ok = ok && cnt[c] <= (uint32_t)kWave;
    return ok;
}

// One light segment of the reduction: the g tile into LDS, the listed
// lane's g picked at its place, its fp64 terms, and g * 0 of every g.
__device__ __forceinline__ void light_tile(float* tile, const float4 (&vg)[kVjpBatchLarge], float d, uint32_t place,
                                           uint32_t rec, double& D, double& G, float& zg, float& g_out)
{
    tile_store(tile, vg);
#pragma unroll
    for (int u = 0; u < kVjpBatchLarge; ++u)
        zg += ((vg[u].x * 0.0f + vg[u].y * 0.0f) + (vg[u].z * 0.0f + vg[u].w * 0.0f));
    __builtin_amdgcn_wave_barrier();
    if ((uint32_t)lane_id() < rec) {
        const float gj = tile[place];
        acc_dg(d, gj, D, G);
        g_out = gj;
    }
    __builtin_amdgcn_wave_barrier();
}

}  // namespace

// Emission with the record, one wave per segment.  A first walk over the
// wave's 16 values per lane evaluates the fp32 density d of each score and
// lists the scores with d >= kDensCut (value index order, lanes ascending)
// in LDS, with their places.  An unlisted score lies more than 27.7 alpha
// from b, so its p is d (left of b) or 1 - d (right of b, 1 in fp32) with
// d < 2^-40: taken from the fp32 d, p is within 1e-18 of the fp64 value, and
// the lane's unlisted scores enter the mass as a count (right of b) plus an
// fp32 sum of their signed d (at most 16 terms below 2^-40 per tile).  The
// listed scores -- about 4% of c4's -- are then evaluated 64 at a time: p
// with the fp64 exponential (as the score-only emission), d again for the
// record's values, which go straight to global memory with their places
// when the segment keeps them.  A last walk picks each lane's listed p out
// of LDS and writes p.  The fp64 arithmetic is thus spent once per 64 listed
// scores, not once per score.
template <bool kNT>
__global__ __launch_bounds__(kStreamThreads) void emit_seg_kernel(EmitArgs a)
{
    constexpr int kB = kVjpBatchLarge;  // one large VJP tile per step (a segment per wave)
    constexpr int kL = kSegScores + kWave;  // the list, then one slot per lane for unlisted scores
    __shared__ double red[kStreamThreads / kWave];
    __shared__ float lst[kStreamThreads / kWave][kL];  // listed scores, then their p
    __shared__ uint16_t lpl[kStreamThreads / kWave][kSegScores];  // places of the listed scores
    Status* st = a.st;
    if (st->solve_state != kSolveOk)
        return;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = wave_index();
    const double b = *a.b;
    const double c = a.log2e_over_alpha;
    const int64_t G = gridDim.x;
    double acc = 0.0;
    const int64_t T = whole_tiles<kB>(a.n);
    const float4* s4 = reinterpret_cast<const float4*>(a.s);
    float4* p4 = reinterpret_cast<float4*>(a.p);
    float* ls = lst[wave];
    uint16_t* lp = lpl[wave];
    for (int64_t t0 = blockIdx.x; t0 < T; t0 += G) {
        const int64_t t = T - 1 - t0;  // descending: see the note above
        const int64_t seg = t * kSegPerTile + wave;
        float4 v[kB];
        load_q<kB>(s4, t, v);
        uint32_t nzb = 0, cnt = 0, n_right = 0;
        float fp[kSegV];      // p of the score if it is not listed
        float far_d = 0.0f;   // unlisted scores' signed d
#pragma unroll
        for (int i = 0; i < kSegV; ++i) {
            const float4 q = v[i / 4];
            const float sv = (i & 3) == 0 ? q.x : (i & 3) == 1 ? q.y : (i & 3) == 2 ? q.z : q.w;
            const bool rt = (double)sv - b > 0.0;
            const float d = dens(sv, b, c);
            const bool nz = d >= kDensCut;
            fp[i] = rt ? 1.0f : d;
            far_d += nz ? 0.0f : (rt ? -d : d);
            n_right += (uint32_t)(!nz && rt);
            nzb |= (uint32_t)nz << i;
            const uint64_t lm = __builtin_amdgcn_ballot_w64(nz);
            // unlisted lanes write a slot of their own past the list (no
            // branch, so each value's work stays in one block, in order)
            const uint32_t at = nz ? cnt + rank_in_mask(lm) : (uint32_t)(kSegScores + lane);
            ls[at] = sv;
            if (nz)
                lp[at] = (uint16_t)((i >> 2) * 256 + lane * 4 + (i & 3));
            cnt += (uint32_t)__popcll(lm);
            __builtin_amdgcn_sched_barrier(0);
        }
        acc += (double)n_right + (double)far_d;  // unlisted scores: p = 1 - d or d
        __builtin_amdgcn_wave_barrier();
        const bool keep = cnt <= (uint32_t)kSegCap;
        uint64_t* ent = a.seg.ent + seg * kSegCap;
        for (uint32_t j = (uint32_t)lane; j < cnt; j += kWave) {
            const float sv = ls[j];
            ls[j] = emit_one(sv, b, c, acc);
            if (keep)
                __builtin_nontemporal_store(seg_entry(dens(sv, b, c), lp[j]), &ent[j]);
        }
        __builtin_amdgcn_wave_barrier();
        uint32_t pre = 0;
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            float o[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int i = 4 * u + h;
                const bool nz = (nzb >> i) & 1u;
                const uint64_t lm = __builtin_amdgcn_ballot_w64(nz);
                const float lpv = ls[nz ? pre + rank_in_mask(lm) : (uint32_t)(kSegScores + lane)];
                o[h] = nz ? lpv : fp[i];
                pre += (uint32_t)__popcll(lm);
            }
            store4<kNT>(&p4[t * (kB * kStreamThreads) + u * kStreamThreads + tid], make_float4(o[0], o[1], o[2], o[3]));
        }
        if (lane == 0)
            __builtin_nontemporal_store(keep ? cnt : kSegDense, &a.seg.cnt[seg]);
        __builtin_amdgcn_wave_barrier();
    }
    for (int64_t i = ragged_start<kB>(a.n, T) + tid; i < a.n; i += kStreamThreads)
        a.p[i] = emit_one(a.s[i], b, c, acc);
    block_sum_to(acc, red, &a.partials[blockIdx.x]);
    if (blockIdx.x == 0 && tid == 0) {
        st->seg_valid = 1u;
        st->seg_n = (uint64_t)a.n;
        st->seg_alpha = a.alpha;
        st->seg_scores = (uint64_t)reinterpret_cast<uintptr_t>(a.s);
    }
}

namespace {

__device__ __forceinline__ bool vjp_seg_usable(const VjpArgs& a)
{
    if (a.fst == nullptr || a.seg.cnt == nullptr)
        return false;
    const Status* f = a.fst;
    return f->seg_valid != 0u && f->b == *a.b && f->seg_n == (uint64_t)a.n && f->seg_alpha == a.alpha &&
           f->seg_scores == (uint64_t)reinterpret_cast<uintptr_t>(a.s);
}

}  // namespace

// (D, G) with the record.  A listed segment: the wave's g tile goes to LDS
// as whole float4, each listed (d, place) pair picks its g there -- one
// fp64 term per listed score -- and the listed g values are stored,
// compacted, for the gradient kernel.  Every g still enters G as g * 0 (an
// fp32 sum, folded in at the end), so a non-finite g makes G non-finite as
// in the score-reading kernel.  A dense segment reads the scores.
__global__ __launch_bounds__(kStreamThreads) void vjp_reduce_seg_kernel(VjpArgs a)
{
    constexpr int kB = kVjpBatchLarge;
    __shared__ double red[2][kStreamThreads / kWave];
    __shared__ float gt[kStreamThreads / kWave][kSegScores];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = wave_index();
    const double b = *a.b;
    const double c = a.log2e_over_alpha;
    const int64_t G = gridDim.x;
    const bool use_seg = vjp_seg_usable(a);
    const int64_t T = whole_tiles<kB>(a.n);
    const float4* s4 = reinterpret_cast<const float4*>(a.s);
    const float4* g4 = reinterpret_cast<const float4*>(a.g);
    float* tile = gt[wave];
    double D = 0.0, G_ = 0.0;
    float zg = 0.0f;  // sum of g * 0 over listed segments: NaN iff some g there is not finite
    for (int64_t tb = blockIdx.x; tb < T; tb += kCntChunk * G) {
        uint32_t cnts[kCntChunk];
        if (use_seg)
            fetch_counts(a, [&](int k) { return tb + (int64_t)k * G; }, T, cnts);
        if (use_seg && chunk_is_light(cnts)) {
            // every segment of the chunk lists at most one value per lane:
            // all (d, place) entries are read at once, and the listed g
            // values are stored at the end, so no store sits between a load
            // and its use
            float dj[kCntChunk], gk[kCntChunk];
            uint32_t pj[kCntChunk];
#pragma unroll
            for (int k = 0; k < kCntChunk; ++k) {
                const int64_t t = tb + (int64_t)k * G;
                const int64_t seg = (t < T ? t : 0) * kSegPerTile + wave;
                const uint64_t e = a.seg.ent[seg * kSegCap + lane];
                dj[k] = entry_d(e);
                pj[k] = entry_place(e);
                gk[k] = 0.0f;
            }
#pragma unroll
            for (int k = 0; k < kCntChunk; ++k) {
                const int64_t t0 = tb + (int64_t)k * G;
                float4 va[kB];
                if (t0 < T) {
                    load_q<kB>(g4, t0, va);
                    light_tile(tile, va, dj[k], pj[k], cnts[k], D, G_, zg, gk[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < kCntChunk; ++k) {
                const int64_t t = tb + (int64_t)k * G;
                if (t < T && (uint32_t)lane < cnts[k])
                    __builtin_nontemporal_store(gk[k], &a.gl[(t * kSegPerTile + wave) * kSegCap + lane]);
            }
            continue;
        }
        for (int k = 0; k < kCntChunk; ++k) {
            const int64_t t = tb + (int64_t)k * G;
            if (t >= T)
                break;
            const uint32_t rec = use_seg ? cnts[k] : kSegDense;
            float4 vg[kB];
            if (rec == kSegDense) {
                float4 vs[kB];
                load_q<kB>(g4, t, vg);
                load_q<kB>(s4, t, vs);
#pragma unroll
                for (int u = 0; u < kB; ++u) {
                    acc_dg(dens(vs[u].x, b, c), vg[u].x, D, G_);
                    acc_dg(dens(vs[u].y, b, c), vg[u].y, D, G_);
                    acc_dg(dens(vs[u].z, b, c), vg[u].z, D, G_);
                    acc_dg(dens(vs[u].w, b, c), vg[u].w, D, G_);
                }
            } else {
                const int64_t seg = t * kSegPerTile + wave;
                const uint64_t* ent = a.seg.ent + seg * kSegCap;
                uint64_t ej[kSegSteps];
                load_q<kB>(g4, t, vg);
#pragma unroll
                for (int q = 0; q < kSegSteps; ++q) {
                    const uint32_t j = (uint32_t)(q * kWave + lane);
                    ej[q] = j < rec ? ent[j] : 0ull;
                }
                float dj[kSegSteps];
                uint32_t pj[kSegSteps];
#pragma unroll
                for (int q = 0; q < kSegSteps; ++q) {
                    dj[q] = entry_d(ej[q]);
                    pj[q] = entry_place(ej[q]);
                }
                tile_store(tile, vg);
#pragma unroll
                for (int u = 0; u < kB; ++u)
                    zg += ((vg[u].x * 0.0f + vg[u].y * 0.0f) + (vg[u].z * 0.0f + vg[u].w * 0.0f));
                __builtin_amdgcn_wave_barrier();
                float* gl = a.gl + seg * kSegCap;
#pragma unroll
                for (int q = 0; q < kSegSteps; ++q) {
                    const uint32_t j = (uint32_t)(q * kWave + lane);
                    if (j < rec) {
                        const float gj = tile[pj[q]];
                        acc_dg(dj[q], gj, D, G_);
                        __builtin_nontemporal_store(gj, &gl[j]);
                    }
                }
                __builtin_amdgcn_wave_barrier();
            }
        }
    }
    for (int64_t i = ragged_start<kB>(a.n, T) + tid; i < a.n; i += kStreamThreads) {
        acc_dg(dens(a.s[i], b, c), a.g[i], D, G_);
    }
    G_ += (double)zg;
    block_sum_to(D, red[0], &a.partials[2 * blockIdx.x]);
    __syncthreads();
    block_sum_to(G_, red[1], &a.partials[2 * blockIdx.x + 1]);
}

// The gradient with the record.  A listed segment: the wave zeroes its LDS
// tile, each listed (d, g, place) triple writes (d/alpha)(g - G/D) at its
// place, and the lanes move the tile out as whole float4.  A dense segment
// reads the scores and g.
template <bool kNT>
__global__ __launch_bounds__(kStreamThreads) void vjp_apply_seg_kernel(VjpArgs a, int32_t reduce_blocks)
{
    constexpr int kB = kVjpBatchLarge;
    __shared__ double red[2][kStreamThreads / kWave];
    __shared__ double tot[2];
    __shared__ float ot[kStreamThreads / kWave][kSegScores];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = wave_index();
    double D = 0.0, G_ = 0.0;
    for (int i = tid; i < reduce_blocks; i += kStreamThreads) {
        D += a.partials[2 * i];
        G_ += a.partials[2 * i + 1];
    }
    block_sum_to(D, red[0], &tot[0]);
    __syncthreads();
    block_sum_to(G_, red[1], &tot[1]);
    __syncthreads();
    const Ratio2 ratio = split_ratio(tot[0] > 0.0 ? tot[1] / tot[0] : 0.0);
    const float inv_alpha = (float)(1.0 / a.alpha);
    const double b = *a.b;
    const double c = a.log2e_over_alpha;
    const int64_t G = gridDim.x;
    // a non-finite g leaves G non-finite: then every g is read, as the
    // score-reading kernel does
    const bool use_seg = vjp_seg_usable(a) && isfinite(tot[1]);
    const int64_t T = whole_tiles<kB>(a.n);
    const float4* s4 = reinterpret_cast<const float4*>(a.s);
    const float4* g4 = reinterpret_cast<const float4*>(a.g);
    float4* o4 = reinterpret_cast<float4*>(a.grad);
    float* tile = ot[wave];
    for (int64_t tb = blockIdx.x; tb < T; tb += kCntChunk * G) {
        // descending tiles: see the note above
        uint32_t cnts[kCntChunk];
        if (use_seg)
            fetch_counts(a, [&](int k) { return T - 1 - (tb + (int64_t)k * G); }, T, cnts);
        if (use_seg && chunk_is_light(cnts)) {
            // every segment of the chunk lists at most one value per lane:
            // all (d, g, place) triples are read at once, then each tile is
            // composed in LDS and stored
            uint64_t ec[kCntChunk];
            float gc[kCntChunk];
#pragma unroll
            for (int k = 0; k < kCntChunk; ++k) {
                const int64_t t0 = tb + (int64_t)k * G;
                const int64_t seg = (t0 < T ? T - 1 - t0 : 0) * kSegPerTile + wave;
                ec[k] = a.seg.ent[seg * kSegCap + lane];
                gc[k] = a.gl[seg * kSegCap + lane];
            }
#pragma unroll
            for (int k = 0; k < kCntChunk; ++k) {
                const int64_t t0 = tb + (int64_t)k * G;
                if (t0 >= T)
                    break;
                const int64_t t = T - 1 - t0;
                float4 o[kB];
#pragma unroll
                for (int u = 0; u < kB; ++u)
                    o[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                tile_store(tile, o);
                __builtin_amdgcn_wave_barrier();
                if ((uint32_t)lane < cnts[k])
                    tile[entry_place(ec[k])] = entry_d(ec[k]) * inv_alpha * minus_ratio(gc[k], ratio);
                __builtin_amdgcn_wave_barrier();
                tile_load(tile, o);
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int u = 0; u < kB; ++u)
                    store4<kNT>(&o4[t * (kB * kStreamThreads) + u * kStreamThreads + tid], o[u]);
            }
            continue;
        }
        for (int k = 0; k < kCntChunk; ++k) {
            const int64_t t0 = tb + (int64_t)k * G;
            if (t0 >= T)
                break;
            const int64_t t = T - 1 - t0;
            const uint32_t rec = use_seg ? cnts[k] : kSegDense;
            float4 o[kB];
            if (rec == kSegDense) {
                float4 vs[kB], vg[kB];
                load_q<kB>(s4, t, vs);
                load_q<kB>(g4, t, vg);
#pragma unroll
                for (int u = 0; u < kB; ++u) {
                    o[u].x = dens(vs[u].x, b, c) * inv_alpha * minus_ratio(vg[u].x, ratio);
                    o[u].y = dens(vs[u].y, b, c) * inv_alpha * minus_ratio(vg[u].y, ratio);
                    o[u].z = dens(vs[u].z, b, c) * inv_alpha * minus_ratio(vg[u].z, ratio);
                    o[u].w = dens(vs[u].w, b, c) * inv_alpha * minus_ratio(vg[u].w, ratio);
                }
            } else {
                const int64_t seg = t * kSegPerTile + wave;
                const uint64_t* ent = a.seg.ent + seg * kSegCap;
                const float* gl = a.gl + seg * kSegCap;
                uint64_t ej[kSegSteps];
                float gj[kSegSteps];
#pragma unroll
                for (int q = 0; q < kSegSteps; ++q) {
                    const uint32_t j = (uint32_t)(q * kWave + lane);
                    ej[q] = j < rec ? ent[j] : 0ull;
                    gj[q] = j < rec ? gl[j] : 0.0f;
                }
                float dj[kSegSteps];
                uint32_t pj[kSegSteps];
#pragma unroll
                for (int q = 0; q < kSegSteps; ++q) {
                    dj[q] = entry_d(ej[q]);
                    pj[q] = entry_place(ej[q]);
                }
#pragma unroll
                for (int u = 0; u < kB; ++u)
                    o[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                tile_store(tile, o);
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int q = 0; q < kSegSteps; ++q) {
                    const uint32_t j = (uint32_t)(q * kWave + lane);
                    if (j < rec)
                        tile[pj[q]] = dj[q] * inv_alpha * minus_ratio(gj[q], ratio);
                }
                __builtin_amdgcn_wave_barrier();
                tile_load(tile, o);
                __builtin_amdgcn_wave_barrier();
            }
#pragma unroll
            for (int u = 0; u < kB; ++u)
                store4<kNT>(&o4[t * (kB * kStreamThreads) + u * kStreamThreads + tid], o[u]);
        }
    }
    for (int64_t i = ragged_start<kB>(a.n, T) + tid; i < a.n; i += kStreamThreads)
        a.grad[i] = dens(a.s[i], b, c) * inv_alpha * minus_ratio(a.g[i], ratio);
}

hipError_t launch_emit(const EmitArgs& a, bool fold_mass, hipStream_t stream)
{
    const bool vec = ((reinterpret_cast<uintptr_t>(a.s) | reinterpret_cast<uintptr_t>(a.p)) & 15u) == 0;
    const dim3 grid(a.blocks), block(kStreamThreads);
    if (!vec)
        STK_LAUNCH(kKEmit, stream, (emit_kernel<1, false, false>), grid, block, 0, stream, a);
    else if (a.seg.cnt != nullptr && a.n >= kSegMinN && a.n >= kNontemporalMin)
        STK_LAUNCH(kKEmit, stream, emit_seg_kernel<true>, grid, block, 0, stream, a);
    else if (a.seg.cnt != nullptr && a.n >= kSegMinN)
        STK_LAUNCH(kKEmit, stream, emit_seg_kernel<false>, grid, block, 0, stream, a);
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
    } else if (a.seg.cnt != nullptr && a.n >= kSegMinN) {
        STK_LAUNCH(kKVjpReduce, stream, vjp_reduce_seg_kernel, gr, block, 0, stream, r);
        if (a.n >= kNontemporalMin)
            STK_LAUNCH(kKVjpApply, stream, vjp_apply_seg_kernel<true>, ga, block, 0, stream, a, r.blocks);
        else
            STK_LAUNCH(kKVjpApply, stream, vjp_apply_seg_kernel<false>, ga, block, 0, stream, a, r.blocks);
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
