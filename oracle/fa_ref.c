/*
 * fa_ref.c -- CPU oracle for the exact attention forward (fp64, plain C).
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg.  The product path never links or calls it.
 *
 * This is the ordinary three-step attention written out for one query row
 * at a time: scores, softmax (with the row maximum subtracted), weighted
 * sum of value vectors.  There is no tiling, no online rescaling and no
 * reordering beyond a plain left-to-right loop.  See fa_ref.h for the
 * formulas and the passages they follow.
 *
 * Parallelism: rows are independent (each has its own maximum, sum and
 * output, as the joelfernandes.org page stresses in "Online softmax, one
 * row at a time"), so an OpenMP loop over rows changes nothing in any
 * row's arithmetic.
 */
#include "fa_ref.h"

#include <math.h>
#include <stdlib.h>
#include <omp.h>

/*
 * One query row.
 *   qi      : the query vector, length d
 *   kh, vh  : the keys and values of this (b, h), [T][d]
 *   n_vis   : number of visible keys; keys 0 .. n_vis-1 are visible
 *             (causal: i+1, otherwise T)
 *   s       : scratch of length >= n_vis
 *   o_row   : output, length d
 *   lse_out : output, one scalar
 */
static void attend_one_row(const double* qi, const double* kh, const double* vh,
                           int64_t n_vis, int64_t d, double scale,
                           double* s, double* o_row, double* lse_out)
{
    /* Step 1: the visible scores s_j = scale * <q_i, k_j>. */
    for (int64_t j = 0; j < n_vis; ++j) {
        const double* kj = kh + j * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += qi[c] * kj[c];
        s[j] = scale * dot;
    }

    /* Step 2: softmax with the row maximum subtracted. */
    double m = -INFINITY;
    for (int64_t j = 0; j < n_vis; ++j)
        if (s[j] > m) m = s[j];

    double l = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        s[j] = exp(s[j] - m);          /* s now holds the unnormalised weights */
        l += s[j];
    }

    /* Step 3: the weighted sum of value vectors, divided by the sum. */
    for (int64_t c = 0; c < d; ++c)
        o_row[c] = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        const double* vj = vh + j * d;
        const double w = s[j];
        for (int64_t c = 0; c < d; ++c)
            o_row[c] += w * vj[c];
    }
    for (int64_t c = 0; c < d; ++c)
        o_row[c] /= l;

    *lse_out = m + log(l);
}

static int sizes_ok(int64_t B, int64_t H, int64_t T, int64_t d)
{
    return B >= 1 && H >= 1 && T >= 1 && d >= 1;
}

int fa_ref_fwd_rows_f64(const double* q, const double* k, const double* v,
                        int64_t B, int64_t H, int64_t T, int64_t d,
                        int causal, double scale,
                        const int64_t* rows, int64_t n_rows,
                        double* o_rows, double* lse_rows)
{
    if (!q || !k || !v || !rows || !o_rows || !lse_rows) return -1;
    if (!sizes_ok(B, H, T, d) || n_rows < 0) return -1;
    const int64_t n_total = B * H * T;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= n_total) return -1;

    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)T * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!s) continue;
            const int64_t flat = rows[r];
            const int64_t bh = flat / T;     /* b*H + h */
            const int64_t i = flat % T;
            const double* kh = k + bh * T * d;
            const double* vh = v + bh * T * d;
            const int64_t n_vis = causal ? i + 1 : T;
            attend_one_row(q + flat * d, kh, vh, n_vis, d, scale, s,
                           o_rows + r * d, lse_rows + r);
        }
        free(s);
    }
    return failed ? -2 : 0;
}

int fa_ref_fwd_f64(const double* q, const double* k, const double* v,
                   double* o, double* lse,
                   int64_t B, int64_t H, int64_t T, int64_t d,
                   int causal, double scale)
{
    if (!q || !k || !v || !o || !lse) return -1;
    if (!sizes_ok(B, H, T, d)) return -1;
    const int64_t n_total = B * H * T;

    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)T * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t flat = 0; flat < n_total; ++flat) {
            if (!s) continue;
            const int64_t bh = flat / T;
            const int64_t i = flat % T;
            const int64_t n_vis = causal ? i + 1 : T;
            attend_one_row(q + flat * d, k + bh * T * d, v + bh * T * d,
                           n_vis, d, scale, s, o + flat * d, lse + flat);
        }
        free(s);
    }
    return failed ? -2 : 0;
}

int fa_ref_num_threads(void)
{
    return omp_get_max_threads();
}
