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

/*
 * The general problem: Hq query heads over Hkv key/value heads (query head h
 * reads key/value head h / (Hq / Hkv): consecutive query heads share one,
 * the grouping of "FlashAttention and Fused Kernels: Attention Without the
 * n x n Matrix", Step 4, for Llama 3.1 8B), Tq query rows over Tk keys.  With
 * causal, the query rows are the last Tq positions of the Tk-long sequence:
 * query i sees keys j <= i + (Tk - Tq) ("Flash Attention, tiled", section
 * "Ordinary causal attention", for Tq = Tk; a decode row, Tq = 1, sees every
 * cached key).  Causal needs Tq <= Tk so that every row sees a key.
 */
static int general_ok(int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d, int causal)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 1 || Tk < 1 || d < 1) return 0;
    if (Hq % Hkv != 0) return 0;
    if (causal && Tq > Tk) return 0;
    return 1;
}

/* Key/value head (b * Hkv + h / group) of flat query row `flat`. */
static int64_t kv_head_of(int64_t flat, int64_t Hq, int64_t Hkv, int64_t Tq)
{
    const int64_t bh = flat / Tq;
    const int64_t b = bh / Hq, h = bh % Hq;
    return b * Hkv + h / (Hq / Hkv);
}

static int64_t visible_of(int64_t flat, int64_t Tq, int64_t Tk, int causal)
{
    const int64_t i = flat % Tq;
    return causal ? i + (Tk - Tq) + 1 : Tk;
}

int fa_ref_attn_rows_f64(const double* q, const double* k, const double* v,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                         int causal, double scale,
                         const int64_t* rows, int64_t n_rows,
                         double* o_rows, double* lse_rows)
{
    if (!q || !k || !v || !rows || !o_rows || !lse_rows) return -1;
    if (!general_ok(B, Hq, Hkv, Tq, Tk, d, causal) || n_rows < 0) return -1;
    const int64_t n_total = B * Hq * Tq;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= n_total) return -1;

    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)Tk * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!s) continue;
            const int64_t flat = rows[r];
            const int64_t kvh = kv_head_of(flat, Hq, Hkv, Tq);
            attend_one_row(q + flat * d, k + kvh * Tk * d, v + kvh * Tk * d,
                           visible_of(flat, Tq, Tk, causal), d, scale, s,
                           o_rows + r * d, lse_rows + r);
        }
        free(s);
    }
    return failed ? -2 : 0;
}

int fa_ref_attn_f64(const double* q, const double* k, const double* v,
                    double* o, double* lse,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                    int causal, double scale)
{
    if (!q || !k || !v || !o || !lse) return -1;
    if (!general_ok(B, Hq, Hkv, Tq, Tk, d, causal)) return -1;
    const int64_t n_total = B * Hq * Tq;

    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)Tk * sizeof(double));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t flat = 0; flat < n_total; ++flat) {
            if (!s) continue;
            const int64_t kvh = kv_head_of(flat, Hq, Hkv, Tq);
            attend_one_row(q + flat * d, k + kvh * Tk * d, v + kvh * Tk * d,
                           visible_of(flat, Tq, Tk, causal), d, scale, s, o + flat * d, lse + flat);
        }
        free(s);
    }
    return failed ? -2 : 0;
}

/* The square problem with one key/value head per query head. */
int fa_ref_fwd_rows_f64(const double* q, const double* k, const double* v,
                        int64_t B, int64_t H, int64_t T, int64_t d,
                        int causal, double scale,
                        const int64_t* rows, int64_t n_rows,
                        double* o_rows, double* lse_rows)
{
    return fa_ref_attn_rows_f64(q, k, v, B, H, H, T, T, d, causal, scale, rows, n_rows, o_rows, lse_rows);
}

int fa_ref_fwd_f64(const double* q, const double* k, const double* v,
                   double* o, double* lse,
                   int64_t B, int64_t H, int64_t T, int64_t d,
                   int causal, double scale)
{
    return fa_ref_attn_f64(q, k, v, o, lse, B, H, H, T, T, d, causal, scale);
}

int fa_ref_num_threads(void)
{
    return omp_get_max_threads();
}
