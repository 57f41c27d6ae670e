/*
 * soft_topk.h -- C ABI of the MI355X (gfx950) LapSum soft top-k library.
 *
 * The operator (gist.science technical summary of "Fast LapSum: Exact
 * Differentiable Top-k at Million Scale", section 2.1 "The LapSum Operator"):
 *
 *     p_i = F((s_i - b) / alpha),   F = standard Laplace CDF,
 *     b   = the unique threshold with  sum_i p_i = k   (0 < k < n, alpha > 0),
 *
 * and its implicit-function vector-Jacobian product (same section: the
 * backward pass is analytic):
 *
 *     d_i = exp(-|s_i - b| / alpha) / 2,   D = sum_i d_i,   G = sum_i g_i d_i,
 *     grad_i = (d_i / alpha) * (g_i - G / D).
 *
 * The forward localises b by probabilistic bracketing (aiqbench.com abstract
 * of Fast LapSum; gist.science summary section 2.2 "Probabilistic
 * Bracketing", steps 1-4): a Philox sample of kernel-noised scores gives a
 * binomial order-statistic bracket [a_L, a_R); one streaming pass folds the
 * scores outside it into tail counts and exponential sums and keeps the band
 * inside it; the band alone is sorted and solved in closed form (section 2.2
 * "Full-Sort Solver"); the bracket is certified exactly, widened when the
 * certificate fails, split at a tied value that floods the band, and a full
 * device radix sort covers the worst case.  Vectors of at most 8192 scores
 * are instead sorted and solved whole by one kernel.  The returned b is the
 * exact root (up to fp64 rounding) whichever route is taken.
 *
 * Conventions shared by every entry point:
 *  - Array pointers (scores, grad_p, out_p, grad_s, b, workspace) are DEVICE
 *    pointers owned by the caller.  The library never allocates device memory.
 *  - scores / p / gradients are fp32, contiguous, length n.  b is fp64.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every kernel is enqueued on it.
 *  - Return value: 0 on success, else one of the SOFT_TOPK_E* codes below.
 *    Arguments are validated on the host before anything is enqueued; on
 *    SOFT_TOPK_EINVAL nothing is launched and the outputs are untouched.
 *  - Limits: 1 <= n <= 2^31 - 1.
 *  - Calls on different streams need distinct workspaces; the library keeps
 *    no other state apart from one small pinned host buffer per host thread
 *    and the 16 KiB per-GPU array of soft_topk_backward_noalloc.
 */
#ifndef SOFT_TOPK_H
#define SOFT_TOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SOFT_TOPK_OK 0
#define SOFT_TOPK_EINVAL 1     /* bad n, k, alpha, pointer, or params      */
#define SOFT_TOPK_ENONFINITE 2 /* a score is NaN or +-Inf                  */
#define SOFT_TOPK_EWORKSPACE 3 /* workspace NULL or smaller than required  */
#define SOFT_TOPK_EHIP 4       /* a HIP runtime call failed                */
#define SOFT_TOPK_ESOLVE 5     /* every route failed its certificate       */

/* Route the forward took (soft_topk_stats.path). */
#define SOFT_TOPK_PATH_BRACKET 1  /* bracket certified on the first pass    */
#define SOFT_TOPK_PATH_WIDENED 2  /* certified after widening the bracket, or
                                     after splitting it at a tied value     */
#define SOFT_TOPK_PATH_FULLSORT 3 /* full device radix sort of all scores   */
#define SOFT_TOPK_PATH_SINGLE 4   /* n <= 8192: one kernel sorts all scores
                                     in registers and solves them exactly   */
#define SOFT_TOPK_PATH_ALL_SCORES 5 /* the band overflowed its buffer (or,
                                     as on the last call on this thread with
                                     the same n, k, alpha and band capacity,
                                     it was expected to and was only
                                     counted); the partition
                                     refinement ran over all n scores and
                                     ended on the exact root                */

/* How a bracketed round solved its band (soft_topk_params.band_route,
 * soft_topk_stats.band_route). */
#define SOFT_TOPK_BAND_DIRECT 1   /* the whole band sorted in one LDS sort     */
#define SOFT_TOPK_BAND_BUCKETS 2  /* value buckets; only the root's is sorted  */
#define SOFT_TOPK_BAND_REFINE 3   /* no sort: partition refinement of the band
                                     (closed form around a split point,
                                     repeated until no score crosses), on one
                                     work-group                              */
#define SOFT_TOPK_BAND_REFINE_STEPS 4 /* the same refinement by step kernels of
                                     many work-groups (larger bands, and all
                                     scores after a band overflow)           */

/* Why a bracketed round was rejected (soft_topk_stats.reject_mask bits). */
#define SOFT_TOPK_REJECT_LOW 1       /* certificate: b lies below a_L        */
#define SOFT_TOPK_REJECT_HIGH 2      /* certificate: b lies at/above a_R     */
#define SOFT_TOPK_REJECT_OVERFLOW 4  /* band larger than its capacity (or
                                        expected to be: only counted)       */
#define SOFT_TOPK_REJECT_BUCKET 8    /* a band bucket too large to sort      */
#define SOFT_TOPK_REJECT_MASS 16     /* post-solve mass check out of bounds  */

/*
 * Tuning and test knobs of the forward.  Pass NULL for the defaults, or fill
 * with soft_topk_default_params() and change fields.  These do not change
 * the result, only the route and its cost (the route-independence of b is
 * what the certificate guarantees).
 */
typedef struct soft_topk_params {
    uint64_t seed;          /* Philox key for the sampler (default 0x5eed)           */
    int32_t samples;        /* sample size m, 1024..262144 (default 65536)            */
    double z;               /* bracket half-width in binomial standard deviations;
                               ranks use exact binomial tails at Phi(-z) (default 5) */
    int64_t band_capacity;  /* max band elements (0 = default: clamp(n/4, 2^16, 2^22)) */
    int32_t max_widen;      /* extra bracketed rounds before the full sort: widenings
                               after a rejected side, and the split of the bracket
                               at a dominant tied value after a band overflow
                               (default 2; 0: straight to the full sort)         */
    int32_t force_path;     /* 0 auto (n <= 8192: SOFT_TOPK_PATH_SINGLE, else the
                               bracketed route); SOFT_TOPK_PATH_BRACKET: the
                               bracketed route at every n; SOFT_TOPK_PATH_FULLSORT:
                               straight to the full sort                         */
    double mass_tolerance;  /* post-solve |sum p - k| bound; <=0 = default
                               (1e-3 + 1e-12 * n)                                    */
    int32_t verify_mass;    /* 1: wait for the certification pass (fp64 sum of p)
                               and reject a b whose mass misses k by more than
                               mass_tolerance; 0 (default): the call returns once
                               the exact bracket certificate is in, and the
                               emission's fp64 partial sums of p are not folded
                               (the pass runs in full whenever stats are
                               requested, and stats.mass is NaN otherwise)      */
    int32_t band_route;     /* 0 auto: refine the unsorted band, on one
                               work-group (SOFT_TOPK_BAND_REFINE) when its
                               expected size n (r_R - r_L) / m is at most
                               10240, else by step kernels (_REFINE_STEPS),
                               which refine every score when the band
                               overflows; a band refinement that does not end
                               sorts the band.  _REFINE_STEPS forces the step
                               kernels; _DIRECT / _BUCKETS force a sorted
                               route: the whole band in one LDS sort (a band
                               over 8192 scores is bucketed), or buckets      */
} soft_topk_params;

/* Host-side record of one forward call (all fields written on success). */
typedef struct soft_topk_stats {
    int32_t path;           /* SOFT_TOPK_PATH_*                                       */
    int32_t rounds;         /* bracketed rounds run (0 on the full sort when forced,
                               and on SOFT_TOPK_PATH_SINGLE)                      */
    int32_t reject_mask;    /* OR of SOFT_TOPK_REJECT_* over rejected rounds          */
    int32_t band_route;     /* SOFT_TOPK_BAND_* of the last bracketed round (0: none) */
    float a_left, a_right;  /* bracket of the last bracketed round (-inf / +inf and
                               n_band = n on SOFT_TOPK_PATH_SINGLE)                */
    int64_t n_left, n_band, n_right; /* scores below / inside / at-or-above it        */
    double mass_at_left;    /* M(a_L) of the last bracketed round (NaN when it
                               refined: its certificate is the refinement's)      */
    double mass_at_right;   /* M(a_R) of the last bracketed round (NaN likewise)      */
    double b;               /* the threshold (also written to out_b on the device)    */
    double mass;            /* fp64 sum of the emitted p (the certification pass)     */
    int32_t refine_passes;  /* passes of the last round's partition refinement (sums
                               at one split point each; 0 when it sorted)          */
    int32_t pad;
} soft_topk_stats;

/* Fill *params with the defaults listed above. */
void soft_topk_default_params(soft_topk_params* params);

/*
 * Bytes of device workspace soft_topk_forward / soft_topk_forward_ex need for
 * n scores (params may be NULL).  Includes the full-sort buffers (two u32
 * arrays of n) so every route fits.  Returns 0 if n is out of range.
 */
size_t soft_topk_workspace_bytes(int64_t n, const soft_topk_params* params);

/*
 * Bytes at the front of a forward workspace (for n scores) that
 * soft_topk_backward_ex reads: the status block and the saturated-segment
 * record (about 1.1 bytes per score from 2^22 scores on, else 256 bytes).
 * A caller that keeps only this prefix of the forward workspace for the
 * backward (a copy, 256-byte aligned, passed as fwd_workspace with this many
 * bytes) gets the same result as with the whole workspace.  0 if n is out of
 * range.
 */
size_t soft_topk_record_bytes(int64_t n);

/* Bytes of device workspace soft_topk_backward needs for n scores. */
size_t soft_topk_backward_workspace_bytes(int64_t n);

/*
 * Forward.  scores: fp32[n] (device).  k: budget, 0 < k < n (real values
 * allowed).  alpha: temperature > 0, finite.  out_p: fp32[n] (device),
 * out_p[i] = F((scores[i] - b)/alpha).  out_b: one fp64 (device) receiving b.
 * workspace: soft_topk_workspace_bytes(n, NULL) bytes of device memory, any
 * contents, 256-byte aligned.
 * Route: up to 8192 scores (by default) one kernel sorts the whole vector in
 * registers and solves it with the full-sort solver of the gist.science
 * summary of Fast LapSum (section 2.2), exactly, with no bracket to certify;
 * larger n take the bracketed route (sample, streaming pass, the band's
 * partition refinement, whose steps certify the bracket; the sorted band
 * routes and the full sort as fallbacks).
 * Synchronisation: enqueues on `stream` and waits (a 256-byte status
 * read-back) until the solve has certified the bracket (or the one-kernel
 * solve has ended), so that the route is settled on return.  b is final in device memory at that point; the
 * emission of p is already enqueued behind it and completes in stream order,
 * so any later work on `stream` sees the final p.  With
 * params->verify_mass = 1 or a stats record, the fp64 mass sum of p is also
 * completed and waited for, and a b whose mass misses k is rejected.
 * Errors: EINVAL / EWORKSPACE before any launch; ENONFINITE if a score is not
 * finite (out_p / out_b then hold no result); EHIP with the HIP status kept
 * for soft_topk_last_hip_error(); ESOLVE should not happen (every route ends
 * in the full sort, whose solve is exact).
 */
int soft_topk_forward(const float* scores, int64_t n, double k, double alpha,
                      float* out_p, double* out_b,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Forward with explicit params (NULL = defaults) and a host stats record
 * (NULL = not wanted).  Same contract as soft_topk_forward. */
int soft_topk_forward_ex(const float* scores, int64_t n, double k, double alpha,
                         float* out_p, double* out_b,
                         void* workspace, size_t workspace_bytes, void* stream,
                         const soft_topk_params* params, soft_topk_stats* stats);

/*
 * Backward (vector-Jacobian product).  grad_p: fp32[n] upstream gradient
 * (device).  scores: the forward's fp32[n].  alpha: the forward's alpha.
 * b: device pointer to the forward's fp64 threshold.  grad_s: fp32[n]
 * (device) receiving (d_i/alpha)(g_i - G/D).  workspace:
 * soft_topk_backward_workspace_bytes(n) bytes of device memory, any contents.
 * Fully asynchronous on `stream` (no host synchronisation).  Up to 8192
 * scores one work-group computes D, G and the gradient in one kernel; larger
 * n take a reduction kernel and a gradient kernel.
 * Errors: EINVAL / EWORKSPACE before any launch; EHIP on a launch failure.
 */
int soft_topk_backward(const float* grad_p, const float* scores, int64_t n,
                       double alpha, const double* b, float* grad_s,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward that may reuse what the forward recorded in its workspace
 * (fwd_workspace, fwd_workspace_bytes: the forward call's workspace, not
 * written since, 256-byte aligned; NULL = none, as soft_topk_backward).
 * Gist.science summary of Fast LapSum, section 2.2: outside a narrow band
 * of scores around b the soft indicator is saturated, and there the fp32
 * density d_i = e^{-|s_i - b|/alpha}/2 is negligible.  From 2^22 scores on
 * (16-byte aligned vectors), the forward's emission, which knows b, records
 * for every 1024-score segment which scores have d_i >= 2^-40
 * (|s_i - b| < 27.7 alpha) and, when at most 256 do, their d_i.  The
 * backward then takes d from that record instead of reading the scores: the
 * other scores enter D and G with d = 0 and get grad = +0.  Leaving them out
 * moves D and G by at most n 2^-40 and no element of the gradient by more
 * than 2^-39 of the largest one.  Every other element is the same fp32
 * arithmetic on the same d_i as soft_topk_backward's.  D and G are fp64 sums
 * split over another number of work-groups, so G/D may differ in its last
 * bits before it is rounded to fp32.  Every g enters G (as g * 0 where d is
 * left out), so a non-finite grad_p makes G non-finite; then every score is
 * read, and the NaN gradient matches soft_topk_backward's.  The record is
 * used only if the forward status in fwd_workspace names these scores
 * (pointer), n, alpha and this b; otherwise the scores are read.  The scores
 * must be unchanged since that forward.  The backward workspace also holds
 * the listed g values between its two kernels.  Errors as
 * soft_topk_backward, plus EWORKSPACE for a misaligned fwd_workspace.
 */
int soft_topk_backward_ex(const float* grad_p, const float* scores, int64_t n,
                          double alpha, const double* b, float* grad_s,
                          const void* fwd_workspace, size_t fwd_workspace_bytes,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, result and errors
 * as soft_topk_backward, whose kernels it runs: up to 8192 scores one
 * work-group; above, the score-reading reduction and gradient kernels, with
 * the reduction's (D, G) partials (at most 1024 work-groups, 16 KiB) in a
 * fixed device array of the library instead of a workspace.  The grid is
 * capped at that size for every n, so every valid n (1 <= n <= 2^31 - 1)
 * fits; a grid above it would return SOFT_TOPK_EWORKSPACE.  The array is
 * per GPU, set up on the first call on each device (its address looked up
 * with the device current) and held until the process ends; calls on one
 * GPU share it and keep the last call's contents, so calls that overlap on
 * one GPU (other streams, other host threads) race and must be ordered by
 * the caller.  The call must be made with the device of `stream` current.
 * Fully asynchronous on `stream`; makes no hipMalloc, hipFree or other
 * allocating call.
 */
int soft_topk_backward_noalloc(const float* grad_p, const float* scores, int64_t n,
                               double alpha, const double* b, float* grad_s,
                               void* stream);

/*
 * Batched rows.  The aiqbench.com abstract and the gist.science summary of
 * Fast LapSum (sections 1 and 2) name expert activation, token routing and
 * attention pruning as the operator's uses: many independent rows, each a
 * soft top-k of its own.  scores: fp32[rows * n_row] (device), row r at
 * scores + r * n_row.  Every row gets its own threshold b_r (out_b: fp64[rows],
 * device) with sum_i F((s_ri - b_r)/alpha) = k, and out_p[r * n_row + i] =
 * F((s_ri - b_r)/alpha); k and alpha are shared by all rows (0 < k < n_row,
 * alpha > 0).  Every row length is solved on the device alone, fully
 * asynchronously on `stream`, with no workspace (workspace may be NULL):
 * each row is refined without a sort (the segment's closed form about a
 * split point, repeated until no score separates the point from its
 * root), several rows per wave up to 2048 scores, one work-group per row
 * above (the row in registers up to 8192 scores, streamed beyond).
 * Accuracy: fp32 exponentials (relative error a few 1e-7) summed in fp32
 * per thread and in fp64 across the row, and a closed form to a few fp32
 * ulps, so b is within about 1e-6 * alpha (the tests see 1e-7) and p
 * within about 1e-7 of the exact values.  A row holding a NaN or an
 * infinite score gets b = NaN and p = NaN; the call still returns OK.
 * Errors: EINVAL before any launch; EHIP on a launch failure.
 */
int soft_topk_rows_forward(const float* scores, int64_t rows, int64_t n_row,
                           double k, double alpha, float* out_p, double* out_b,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of the batched rows: grad_s[r * n_row + i] =
 * (d_ri/alpha)(g_ri - G_r/D_r) with each row's own D_r and G_r, as in
 * soft_topk_backward (b: the forward's out_b).  No workspace (may be NULL);
 * fully asynchronous: several rows per wave up to 1024 scores, one
 * work-group per row above (streamed beyond 8192).  Errors as
 * soft_topk_rows_forward.
 */
int soft_topk_rows_backward(const float* grad_p, const float* scores, int64_t rows,
                            int64_t n_row, double alpha, const double* b,
                            float* grad_s, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Workspace bytes for the batched calls: always 0 (none needed; kept so
 * callers that size a workspace need not special-case the batched calls). */
size_t soft_topk_rows_workspace_bytes(int64_t rows, int64_t n_row);

/*
 * DFTopK comparator.  The mlsanity.com page "Differentiable Fast Top-K
 * Selection for Large-Scale Recommendation" (abstract) and the gist.science
 * summary of Fast LapSum (section 2.3, "Relation to DFTopK") describe DFTopK
 * as fixing the threshold at the midpoint of the k-th and (k+1)-th largest
 * scores, LapSum's zero-temperature limit, which lets the selected mass
 * drift from k at a finite temperature.  This call computes that operator
 * for comparison: b = (x_(k) + x_(k+1)) / 2 in fp64 (x_(j) the j-th largest
 * score, out_b one fp64, device) and out_p[i] = F((scores[i] - b)/alpha)
 * (fp32, device), F the standard Laplace CDF, with the same emission as
 * soft_topk_forward.  out_mass (one fp64, device; NULL = not wanted)
 * receives sum_i p_i in fp64, whose distance from k is the drift.  k must be
 * a whole number with 1 <= k <= n - 1 (2 <= n <= 2^31 - 1); alpha > 0.
 * workspace: soft_topk_dftopk_workspace_bytes(n) bytes, 256-byte aligned.
 * Route: an exact radix selection of the two order statistics, three
 * streaming passes over the scores (11, 11 and 10 key bits), then the
 * emission; fully asynchronous on `stream` (no host synchronisation).  A NaN
 * score makes b, every p and the mass NaN (no error code, since nothing is
 * read back); infinite scores are ordered like any other value.  There is
 * no backward for this comparator.  Errors: EINVAL / EWORKSPACE before any
 * launch; EHIP on a launch failure.
 */
int soft_topk_dftopk_forward(const float* scores, int64_t n, double k, double alpha,
                             float* out_p, double* out_b, double* out_mass,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of soft_topk_dftopk_forward (0 for n outside [2, 2^31 - 1]). */
size_t soft_topk_dftopk_workspace_bytes(int64_t n);

/*
 * Threshold curve.  The gist.science summary of Fast LapSum (section 2.2,
 * "Full-Sort Solver") reads the root off the masses at the sorted scores;
 * this call returns them.  scores: fp32[n] (device); alpha > 0, finite.
 * out_sorted: fp32[n] (device), the scores in ascending order (-0 returned
 * as +0: the sort keys equal values alike).  out_mass:
 * fp64[n] (device), out_mass[j] = sum_i F((scores[i] - out_sorted[j])/alpha),
 * the k that the threshold b = out_sorted[j] selects (non-increasing in j;
 * for any 0 < k < n the forward's b lies in the gap where it crosses k).
 * workspace: soft_topk_workspace_bytes(n, NULL) bytes (the forward's size),
 * 256-byte aligned.  Route: the full device radix sort, summaries of
 * 4096-score tiles, then the anchored prefix/suffix sums of every value.
 * Synchronisation: one 256-byte status read-back (the score range, which
 * decides the radix passes); the rest is enqueued on `stream`.
 * Errors: EINVAL / EWORKSPACE before any launch; ENONFINITE if a score is not
 * finite (the outputs then hold no result); EHIP on a HIP failure.
 */
int soft_topk_threshold_curve(const float* scores, int64_t n, double alpha, float* out_sorted,
                              double* out_mass, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Text for a return code. */
const char* soft_topk_strerror(int code);

/* The HIP status (hipError_t as int) behind the last EHIP on this thread. */
int soft_topk_last_hip_error(void);

/*
 * Host rank arithmetic of the bracket (exposed for tests; no GPU needed).
 * For m samples of a law whose target quantile is q = 1 - k/n, returns the
 * 1-based ranks r_left < r_right such that the order statistics Y_(r_left) and
 * Y_(r_right) bracket the q-quantile except with probability
 * Phi(-z) on each side under the Binomial(m, q) law of the count of samples at
 * or below it.  r_left = 0 means -inf, r_right = m + 1 means +inf.
 */
int soft_topk_bracket_ranks(int64_t m, double q, double z,
                            int64_t* r_left, int64_t* r_right);

/*
 * Diagnostic: run only the sampler on `scores` and write the m kernel-noised
 * samples Y_j = s[I_j] + alpha * E_j (fp32, device) to out_samples, where
 * (I_j, E_j) come from Philox4x32-10 with counter (j, 0, 0, 0) and key
 * (seed low word, seed high word): I_j = floor(((hi32 << 32 | lo32) * n) / 2^64)
 * from output words 0 (lo32) and 1 (hi32), E_j the Laplace(0,1) inverse CDF
 * of u = (word2 + 0.5) / 2^32.  Asynchronous on `stream`.
 */
int soft_topk_debug_sample(const float* scores, int64_t n, double alpha,
                           uint64_t seed, int32_t m, float* out_samples,
                           void* stream);

/*
 * Diagnostic kernel timing.  soft_topk_profile_begin(mask) makes the library
 * record a HIP event pair on the launch stream around every later launch of
 * each kernel whose bit is set in `mask` (bit i = kernel id i, names from
 * soft_topk_profile_kernel_name); soft_topk_profile_end waits for those
 * events and writes, per kernel id, the summed milliseconds and the launch
 * count into caller arrays of soft_topk_profile_kernel_count() entries
 * (either may be NULL), then stops recording.  Process-wide; not meant for
 * concurrent use from several threads.
 */
int soft_topk_profile_kernel_count(void);
const char* soft_topk_profile_kernel_name(int id);
int soft_topk_profile_begin(uint32_t kernel_mask);
int soft_topk_profile_end(double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* SOFT_TOPK_H */
