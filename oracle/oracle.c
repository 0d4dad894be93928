/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the fp32 sum
 * reduction.  TEST INFRASTRUCTURE ONLY: it is loaded by the test suite, by the
 * smoke check and by the benchmark's CPU-baseline leg, never by the library.
 * It shares no code, header or constant with the GPU path.
 *
 * What is computed is the plain definition of a sum; the pages never fix a
 * summation order, so none is imitated here:
 *
 *   full reduce  S = sum_{i<n} x[i]
 *       ("High-Performance Reduction Kernels" README: a 1D float32 sum of
 *        n elements; "Seven-step reduction: 30x from one kernel": sum is the
 *        first reduction it names)
 *
 *   axis reduce  out[o][i] = sum_{r<R} x[o][r][i]   over a contiguous
 *                [outer, R, inner] array
 *       (POPCORNBENCH Kimi-K2.6 level-1 problem 47 trace, "sum over a
 *        dimension": shape [batch, dim1, dim2] reduced over dim 1, output
 *        element (o, i) at o*inner + i, each one the sum of the R values that
 *        sit inner elements apart)
 *
 * Every fp32 input is widened exactly to fp64 and accumulated in fp64, one
 * element after the other in increasing index order (r increasing for the
 * axis reduce).  Alongside each sum the oracle returns A = sum |x| over the
 * same elements, which is what the acceptance bound |gpu - S| <= 1e-5*A + 1e-6
 * is measured against.  IEEE semantics throughout: no fast-math, no
 * contraction (built with -O2 -ffp-contract=off), NaN and Inf propagate, the
 * empty sum is +0.0.
 *
 * The worst-case error of a sequential fp64 sum of n terms is below
 * (n-1) * 2^-53 * A, i.e. 1.2e-7 * A at n = 1e9: two orders of magnitude under
 * the acceptance bound.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of OpenMP threads a parallel region uses by default. */
int oracle_default_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Full reduce of n floats: one sequential fp64 loop. */
void oracle_sum_1d(const float* x, int64_t n, double* sum, double* abs_sum)
{
    double s = 0.0;
    double a = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double v = (double)x[i];
        s += v;
        a += fabs(v);
    }
    *sum = s;
    *abs_sum = a;
}

/*
 * Axis reduce of a contiguous [outer, R, inner] float array into
 * out[outer * inner] (and abs_out, same layout).  For one output (o, i) the
 * terms are added in increasing r.  The loop over i sits inside the loop over
 * r only so that rows are read front to back; it does not change the order in
 * which any single output receives its terms.  Different o are independent
 * and are shared out over `nthreads` OpenMP threads (<= 0: OpenMP default).
 * Each thread accumulates one o at a time in buffers of its own and then
 * copies them out, so that threads never write the same cache line while
 * they add (with inner == 1, neighbouring o share lines of `out`).
 */
void oracle_sum_dim(const float* x, int64_t outer, int64_t R, int64_t inner,
                    double* out, double* abs_out, int nthreads)
{
    if (nthreads < 1)
        nthreads = oracle_default_threads();
#pragma omp parallel num_threads(nthreads)
    {
        double* s = (double*)malloc((size_t)(inner > 0 ? inner : 1) * sizeof(double));
        double* a = (double*)malloc((size_t)(inner > 0 ? inner : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t o = 0; o < outer; ++o) {
            if (!s || !a) {  /* no buffer: report NaN rather than a wrong sum */
                for (int64_t i = 0; i < inner; ++i)
                    out[o * inner + i] = abs_out[o * inner + i] = NAN;
                continue;
            }
            for (int64_t i = 0; i < inner; ++i) {
                s[i] = 0.0;
                a[i] = 0.0;
            }
            for (int64_t r = 0; r < R; ++r) {
                const float* row = x + (o * R + r) * inner;
                for (int64_t i = 0; i < inner; ++i) {
                    double v = (double)row[i];
                    s[i] += v;
                    a[i] += fabs(v);
                }
            }
            memcpy(out + o * inner, s, (size_t)inner * sizeof(double));
            memcpy(abs_out + o * inner, a, (size_t)inner * sizeof(double));
        }
        free(s);
        free(a);
    }
}

/*
 * The same definition evaluated for m chosen outputs (o_idx[k], i_idx[k]),
 * one at a time, straight from the formula.  Used to check sampled outputs of
 * full-size inputs without reducing the whole array.
 */
void oracle_sum_dim_at(const float* x, int64_t outer, int64_t R, int64_t inner,
                       const int64_t* o_idx, const int64_t* i_idx, int64_t m,
                       double* out, double* abs_out)
{
    (void)outer;
    for (int64_t k = 0; k < m; ++k) {
        const int64_t o = o_idx[k];
        const int64_t i = i_idx[k];
        double s = 0.0;
        double a = 0.0;
        for (int64_t r = 0; r < R; ++r) {
            double v = (double)x[(o * R + r) * inner + i];
            s += v;
            a += fabs(v);
        }
        out[k] = s;
        abs_out[k] = a;
    }
}

/*
 * Other reductions on the same shapes ("Seven-step reduction: 30x from one
 * kernel", opening section: sum, max, the softmax denominator, the L2 norm
 * and the attention row-sum are all the same primitive):
 *
 *   op 1  sum of squares  S = sum x^2   (the L2 norm is its square root)
 *   op 2  maximum         S = max x
 *   op 3  minimum         S = min x
 *
 * (op 0, the sum itself, is oracle_sum_1d / oracle_sum_dim above.)  The
 * square of a widened fp32 value is exact in fp64 (48 significant bits), so
 * the sum of squares is accumulated like the sum, with A = S.  Maximum and
 * minimum follow IEEE 754-2019 maximum / minimum: a NaN anywhere gives NaN,
 * and -0 counts as less than +0, so the result does not depend on the order
 * of the operands.  The maximum of nothing is -Inf, the minimum +Inf; for
 * them A = |S|.  An op outside 1..3 gives NaN.
 */
static double maximum754(double m, double v)
{
    if (isnan(m) || isnan(v))
        return NAN;
    if (m == v)
        return signbit(m) ? v : m; /* +0 over -0 */
    return v > m ? v : m;
}

static double minimum754(double m, double v)
{
    if (isnan(m) || isnan(v))
        return NAN;
    if (m == v)
        return signbit(m) ? m : v; /* -0 over +0 */
    return v < m ? v : m;
}

static double reduce_start(int op)
{
    if (op == 2)
        return -INFINITY;
    if (op == 3)
        return INFINITY;
    return 0.0;
}

/* One term into (s, a) for op 1..3. */
static void reduce_step(int op, double v, double* s, double* a)
{
    if (op == 1) {
        *s += v * v;
        *a += v * v;
    } else if (op == 2) {
        *s = maximum754(*s, v);
    } else if (op == 3) {
        *s = minimum754(*s, v);
    } else {
        *s = NAN;
    }
}

static double reduce_magnitude(int op, double s, double a)
{
    return op == 1 ? a : fabs(s);
}

/* Full reduce of n floats with op 1..3, in index order. */
void oracle_reduce_1d(const float* x, int64_t n, int op, double* res, double* abs_res)
{
    double s = reduce_start(op);
    double a = 0.0;
    for (int64_t i = 0; i < n; ++i)
        reduce_step(op, (double)x[i], &s, &a);
    *res = s;
    *abs_res = reduce_magnitude(op, s, a);
}

/* Axis reduce with op 1..3; same layout and threading as oracle_sum_dim. */
void oracle_reduce_dim(const float* x, int64_t outer, int64_t R, int64_t inner, int op,
                       double* out, double* abs_out, int nthreads)
{
    if (nthreads < 1)
        nthreads = oracle_default_threads();
#pragma omp parallel num_threads(nthreads)
    {
        double* s = (double*)malloc((size_t)(inner > 0 ? inner : 1) * sizeof(double));
        double* a = (double*)malloc((size_t)(inner > 0 ? inner : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t o = 0; o < outer; ++o) {
            if (!s || !a) {
                for (int64_t i = 0; i < inner; ++i)
                    out[o * inner + i] = abs_out[o * inner + i] = NAN;
                continue;
            }
            for (int64_t i = 0; i < inner; ++i) {
                s[i] = reduce_start(op);
                a[i] = 0.0;
            }
            for (int64_t r = 0; r < R; ++r) {
                const float* row = x + (o * R + r) * inner;
                for (int64_t i = 0; i < inner; ++i)
                    reduce_step(op, (double)row[i], &s[i], &a[i]);
            }
            for (int64_t i = 0; i < inner; ++i) {
                out[o * inner + i] = s[i];
                abs_out[o * inner + i] = reduce_magnitude(op, s[i], a[i]);
            }
        }
        free(s);
        free(a);
    }
}

/* The same for m chosen outputs, each straight from the definition. */
void oracle_reduce_dim_at(const float* x, int64_t outer, int64_t R, int64_t inner, int op,
                          const int64_t* o_idx, const int64_t* i_idx, int64_t m,
                          double* out, double* abs_out)
{
    (void)outer;
    for (int64_t k = 0; k < m; ++k) {
        double s = reduce_start(op);
        double a = 0.0;
        for (int64_t r = 0; r < R; ++r)
            reduce_step(op, (double)x[(o_idx[k] * R + r) * inner + i_idx[k]], &s, &a);
        out[k] = s;
        abs_out[k] = reduce_magnitude(op, s, a);
    }
}

/*
 * Cumulative sum along the middle axis of a contiguous [outer, R, inner]
 * array, out having the same shape (POPCORNBENCH level-1 problem 91 trace:
 * y = cumsum(x.flip(1), 1).flip(1), which it spells out as
 * y[i][j] = x[i][j] + x[i][j+1] + ... + x[i][N-1]).
 *   reverse != 0:  out[o][r][i] = sum_{k = r .. R-1} x[o][k][i]
 *   reverse == 0:  out[o][r][i] = sum_{k = 0 .. r}   x[o][k][i]
 * Each output is accumulated in fp64 in the order the definition walks:
 * from the far end of the row (k = R-1 for the reverse sum, k = 0 for the
 * forward one) toward r, one term at a time; abs_out gets the same sums of
 * |x|.  Different (o, i) are independent and shared out over OpenMP threads.
 */
void oracle_cumsum_dim(const float* x, int64_t outer, int64_t R, int64_t inner, int reverse,
                       double* out, double* abs_out, int nthreads)
{
    if (nthreads < 1)
        nthreads = oracle_default_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t o = 0; o < outer; ++o) {
        for (int64_t i = 0; i < inner; ++i) {
            double s = 0.0;
            double a = 0.0;
            for (int64_t k = 0; k < R; ++k) {
                const int64_t r = reverse ? R - 1 - k : k;
                const int64_t e = (o * R + r) * inner + i;
                double v = (double)x[e];
                s += v;
                a += fabs(v);
                out[e] = s;
                abs_out[e] = a;
            }
        }
    }
}

/*
 * Softmax denominator along the middle axis of a contiguous [outer, R, inner]
 * array ("Seven-step reduction: 30x from one kernel", opening section: the
 * softmax denominator is one of the reductions it names).  softmax(x)_r is
 * exp(x_r) / sum_k exp(x_k); written with a shift c that keeps every
 * exponent at or below zero, the denominator is exp(c) * s.  For each output
 * (o, i), over its terms x_r = x[o][r][i], r < R:
 *
 *   m = max_r x_r         (IEEE 754-2019 maximum as above; -Inf for R = 0)
 *   c = m when m is finite, else 0
 *   s = sum_r exp(x_r - c)
 *
 * so that softmax(x)_r = exp(x_r - c) / s and log sum_r exp(x_r) = c + log s.
 * Shifting by 0 when the maximum is infinite is the reading taken for the
 * cases the softmax leaves open: all terms -Inf (or none) give s = 0, a +Inf
 * term gives s = +Inf, a NaN gives NaN.  m_out receives m (exact), s_out
 * receives s: the maximum in a first sweep over r, then exp() of libm in fp64
 * on the exactly widened terms, added in increasing r.  All terms of s are
 * non-negative, so s is also its own magnitude (the acceptance bound's A).
 * Different o are shared out over OpenMP threads.
 */
static double softmax_shift(double m)
{
    return isfinite(m) ? m : 0.0;
}

void oracle_softmax_denom_dim(const float* x, int64_t outer, int64_t R, int64_t inner,
                              double* m_out, double* s_out, int nthreads)
{
    if (nthreads < 1)
        nthreads = oracle_default_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t o = 0; o < outer; ++o) {
        for (int64_t i = 0; i < inner; ++i) {
            double m = -INFINITY;
            for (int64_t r = 0; r < R; ++r)
                m = maximum754(m, (double)x[(o * R + r) * inner + i]);
            const double c = softmax_shift(m);
            double s = 0.0;
            for (int64_t r = 0; r < R; ++r)
                s += exp((double)x[(o * R + r) * inner + i] - c);
            m_out[o * inner + i] = m;
            s_out[o * inner + i] = s;
        }
    }
}

/* The same for m chosen outputs (o_idx[k], i_idx[k]). */
void oracle_softmax_denom_dim_at(const float* x, int64_t outer, int64_t R, int64_t inner,
                                 const int64_t* o_idx, const int64_t* i_idx, int64_t cnt,
                                 double* m_out, double* s_out)
{
    (void)outer;
    for (int64_t k = 0; k < cnt; ++k) {
        const float* col = x + o_idx[k] * R * inner + i_idx[k];
        double m = -INFINITY;
        for (int64_t r = 0; r < R; ++r)
            m = maximum754(m, (double)col[r * inner]);
        const double c = softmax_shift(m);
        double s = 0.0;
        for (int64_t r = 0; r < R; ++r)
            s += exp((double)col[r * inner] - c);
        m_out[k] = m;
        s_out[k] = s;
    }
}
