/*
 * softtopk_oracle.c -- plain fp64 CPU oracle for the LapSum soft top-k operator.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference against
 * which the HIP path is checked.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header, table
 * or helper with the GPU library, and it never calls it.
 *
 * What it computes (sources: the gist.science technical summary of
 * "Fast LapSum: Exact Differentiable Top-k at Million Scale", section 2.1
 * "The LapSum Operator" and section 2.2 "Full-Sort Solver"):
 *
 *   F(x)   = standard Laplace CDF: exp(x)/2 for x <= 0, 1 - exp(-x)/2 for x > 0
 *   M(b)   = sum_i F((s_i - b)/alpha)          (strictly decreasing in b)
 *   b      = the unique root of M(b) = k,  0 < k < n, alpha > 0
 *   p_i    = F((s_i - b)/alpha)
 *   VJP    : d_i = exp(-|s_i - b|/alpha)/2, D = sum d, G = sum g_i d_i,
 *            grad_i = (d_i/alpha) (g_i - G/D)   (G/D taken in scale-free form)
 *            (implicit differentiation of M(b) = k; section 2.1 states the
 *            backward pass is analytic.)
 *
 * The solver follows the full-sort route of section 2.2, in that order:
 * sort the scores, run one numerically stable prefix and one suffix scan of
 * shifted exponential sums (the "threshold curve"), evaluate the mass at every
 * breakpoint, look up the gap where the budget balances, and take the closed
 * form root inside it.  Everything is fp64; the sort is the C library's qsort.
 *
 * Parity is pinned by tests (brute-force bisection, closed forms, the
 * zero-temperature limit, invariances, finite differences); no function here
 * is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENONFINITE 2
#define ORACLE_ENOMEM 5

/* Standard Laplace CDF (the sigma of section 2.1). */
static double laplace_cdf(double x)
{
    if (x <= 0.0)
        return 0.5 * exp(x);
    return 1.0 - 0.5 * exp(-x);
}

static int cmp_double(const void* a, const void* b)
{
    double x = *(const double*)a, y = *(const double*)b;
    return (x > y) - (x < y);
}

static int check_args(const double* s, int64_t n, double k, double alpha)
{
    if (s == NULL || n < 1)
        return ORACLE_EINVAL;
    if (!(alpha > 0.0) || !isfinite(alpha))
        return ORACLE_EINVAL;
    if (!(k > 0.0) || !(k < (double)n))
        return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(s[i]))
            return ORACLE_ENONFINITE;
    return ORACLE_OK;
}

/* Selected mass M(b) = sum_i F((s_i - b)/alpha), straight from the definition. */
double oracle_mass(const double* s, int64_t n, double b, double alpha)
{
    double m = 0.0;
    for (int64_t i = 0; i < n; ++i)
        m += laplace_cdf((s[i] - b) / alpha);
    return m;
}

/*
 * Closed-form root inside the gap [x_lo, x_hi] (section 2.2: once the gap
 * between two sorted scores where the mass crosses k is known, the root in it
 * has a closed form).  With v = exp((x_lo - b)/alpha), w = exp((b - x_hi)/alpha),
 * v*w = g = exp(-(x_hi - x_lo)/alpha), the mass in the gap is
 *     M(b) = A v / 2 + C - B w / 2
 * where A = sum_{x_i <= x_lo} exp((x_i - x_lo)/alpha),
 *       B = sum_{x_i >= x_hi} exp(-(x_i - x_hi)/alpha),
 *       C = number of scores at or above x_hi.
 * M(b) = k is a quadratic in v (or in w); c = C - k picks the root form that
 * has no cancellation, and c = 0 uses the log form, which stays finite when
 * g underflows.
 */
static double gap_root(double x_lo, double x_hi, double A, double B, double c,
                       double alpha)
{
    if (c == 0.0)
        return 0.5 * (x_lo + x_hi) + 0.5 * alpha * log(A / B);
    double g = exp(-(x_hi - x_lo) / alpha);
    double r = sqrt(c * c + A * B * g);
    if (c > 0.0)
        return x_hi + alpha * log((c + r) / B);
    return x_lo - alpha * log((-c + r) / A);
}

/*
 * Threshold b with M(b) = k.  Steps of the full-sort solver:
 *  1. x = sort(s) ascending.
 *  2. prefix scan  A_j = 1 + A_{j-1} exp((x_{j-1} - x_j)/alpha),  A_0 = 1
 *     suffix scan  B_j = 1 + B_{j+1} exp((x_j - x_{j+1})/alpha),  B_{n-1} = 1
 *     (A_j = sum_{i<=j} exp((x_i-x_j)/alpha), B_j = sum_{i>=j} exp(-(x_i-x_j)/alpha);
 *      every factor is <= 1, so nothing overflows for any alpha).
 *  3. breakpoint mass  M(x_j) = A_j/2 + (n-1-j) - B_{j+1} exp(-(x_{j+1}-x_j)/alpha)/2,
 *     M(x_{n-1}) = A_{n-1}/2.
 *  4. locate the gap: root below x_0, above x_{n-1}, or in [x_j, x_{j+1}] with
 *     j the last index whose breakpoint mass is >= k (binary search; the
 *     breakpoint mass is non-increasing in j).
 *  5. closed-form root in that gap.
 */
int oracle_threshold(const double* s, int64_t n, double k, double alpha,
                     double* b_out)
{
    int rc = check_args(s, n, k, alpha);
    if (rc != ORACLE_OK)
        return rc;
    if (b_out == NULL)
        return ORACLE_EINVAL;

    double* x = (double*)malloc(sizeof(double) * (size_t)n);
    double* A = (double*)malloc(sizeof(double) * (size_t)n);
    double* B = (double*)malloc(sizeof(double) * (size_t)(n + 1));
    if (!x || !A || !B) {
        free(x); free(A); free(B);
        return ORACLE_ENOMEM;
    }

    /* 1. sort */
    memcpy(x, s, sizeof(double) * (size_t)n);
    qsort(x, (size_t)n, sizeof(double), cmp_double);

    /* 2. stable prefix and suffix scans */
    A[0] = 1.0;
    for (int64_t j = 1; j < n; ++j)
        A[j] = 1.0 + A[j - 1] * exp((x[j - 1] - x[j]) / alpha);
    B[n] = 0.0;
    B[n - 1] = 1.0;
    for (int64_t j = n - 2; j >= 0; --j)
        B[j] = 1.0 + B[j + 1] * exp((x[j] - x[j + 1]) / alpha);

    /* 3. breakpoint mass, as a function of the breakpoint index */
#define BREAK_MASS(j)                                                        \
    ((j) == n - 1 ? 0.5 * A[n - 1]                                           \
                  : 0.5 * A[(j)] + (double)(n - 1 - (j))                     \
                        - 0.5 * B[(j) + 1] * exp(-(x[(j) + 1] - x[(j)]) / alpha))

    double b;
    if (BREAK_MASS(0) < k) {
        /* root below every score: M(b) = n - B_0 exp((b - x_0)/alpha)/2 */
        b = x[0] + alpha * log(2.0 * ((double)n - k) / B[0]);
    } else if (BREAK_MASS(n - 1) >= k) {
        /* root at or above every score: M(b) = A_{n-1} exp((x_{n-1} - b)/alpha)/2 */
        b = x[n - 1] - alpha * log(2.0 * k / A[n - 1]);
    } else {
        /* 4. last j with M(x_j) >= k; invariant: M(x_lo) >= k > M(x_hi) */
        int64_t lo = 0, hi = n - 1;
        while (hi - lo > 1) {
            int64_t mid = lo + (hi - lo) / 2;
            if (BREAK_MASS(mid) >= k)
                lo = mid;
            else
                hi = mid;
        }
        /* 5. closed form in [x_lo, x_lo+1] */
        double c = (double)(n - 1 - lo) - k;
        b = gap_root(x[lo], x[lo + 1], A[lo], B[lo + 1], c, alpha);
    }
#undef BREAK_MASS

    free(x);
    free(A);
    free(B);
    *b_out = b;
    return ORACLE_OK;
}

/*
 * DFTopK comparator (mlsanity.com page "Differentiable Fast Top-K Selection
 * for Large-Scale Recommendation", abstract; gist.science summary of Fast
 * LapSum, section 2.3 "Relation to DFTopK"): the threshold is fixed at the
 * midpoint of the k-th and (k+1)-th largest scores instead of solving
 * M(b) = k, so the selected mass sum_i F((s_i - b)/alpha) may differ from k.
 * k must be a whole number with 1 <= k <= n - 1.  Sort ascending; the k-th
 * largest is x[n-k] and the (k+1)-th largest x[n-k-1].
 */
int oracle_dftopk_threshold(const double* s, int64_t n, double k, double* b_out)
{
    if (s == NULL || b_out == NULL || n < 2)
        return ORACLE_EINVAL;
    if (!(k >= 1.0) || !(k <= (double)(n - 1)) || k != floor(k))
        return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(s[i]))
            return ORACLE_ENONFINITE;
    double* x = (double*)malloc(sizeof(double) * (size_t)n);
    if (!x)
        return ORACLE_ENOMEM;
    memcpy(x, s, sizeof(double) * (size_t)n);
    qsort(x, (size_t)n, sizeof(double), cmp_double);
    const int64_t kk = (int64_t)k;
    *b_out = 0.5 * (x[n - kk] + x[n - kk - 1]);
    free(x);
    return ORACLE_OK;
}

/* DFTopK forward: its threshold and p_i = F((s_i - b)/alpha). */
int oracle_dftopk_forward(const double* s, int64_t n, double k, double alpha,
                          double* p_out, double* b_out)
{
    if (p_out == NULL || b_out == NULL)
        return ORACLE_EINVAL;
    if (!(alpha > 0.0) || !isfinite(alpha))
        return ORACLE_EINVAL;
    double b;
    int rc = oracle_dftopk_threshold(s, n, k, &b);
    if (rc != ORACLE_OK)
        return rc;
    for (int64_t j = 0; j < n; ++j)
        p_out[j] = laplace_cdf((s[j] - b) / alpha);
    *b_out = b;
    return ORACLE_OK;
}

/* Forward: b and p_i = F((s_i - b)/alpha), in the original order. */
int oracle_forward(const double* s, int64_t n, double k, double alpha,
                   double* p_out, double* b_out)
{
    if (p_out == NULL || b_out == NULL)
        return ORACLE_EINVAL;
    double b;
    int rc = oracle_threshold(s, n, k, alpha, &b);
    if (rc != ORACLE_OK)
        return rc;
    for (int64_t i = 0; i < n; ++i)
        p_out[i] = laplace_cdf((s[i] - b) / alpha);
    *b_out = b;
    return ORACLE_OK;
}

/*
 * Backward (vector-Jacobian product) at a given threshold b.
 * Differentiating sum_j F((s_j - b)/alpha) = k gives db/ds_l = d_l / D, so
 * dp_i/ds_l = (d_i/alpha)(delta_il - d_l/D) and
 * grad_l = sum_i g_i dp_i/ds_l = (d_l/alpha)(g_l - G/D).
 * G/D is a weighted mean of g with weights d_i; the common factor
 * exp(-delta/alpha), delta = min_i |s_i - b|, cancels from it, so it is taken
 * with weights w_i = exp(-(|s_i - b| - delta)/alpha) <= 1 (at least one equals
 * 1), which stays finite when every d_i underflows.
 */
int oracle_backward(const double* g, const double* s, int64_t n, double alpha,
                    double b, double* grad_out)
{
    if (g == NULL || s == NULL || grad_out == NULL || n < 1)
        return ORACLE_EINVAL;
    if (!(alpha > 0.0) || !isfinite(alpha) || !isfinite(b))
        return ORACLE_EINVAL;
    double delta = fabs(s[0] - b);
    for (int64_t i = 1; i < n; ++i)
        if (fabs(s[i] - b) < delta)
            delta = fabs(s[i] - b);
    double W = 0.0, GW = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double w = exp(-(fabs(s[i] - b) - delta) / alpha);
        W += w;
        GW += g[i] * w;
    }
    double ratio = GW / W;
    for (int64_t i = 0; i < n; ++i) {
        double d = 0.5 * exp(-fabs(s[i] - b) / alpha);
        grad_out[i] = (d / alpha) * (g[i] - ratio);
    }
    return ORACLE_OK;
}
