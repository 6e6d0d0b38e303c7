/*
 * fa_ref.c -- CPU oracle for the exact attention forward and backward (fp64, plain C).
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

/*
 * Backward.  The gradients of O = softmax(scale * Q K^T [+ causal mask]) V
 * with respect to Q, K and V for an upstream gradient dO, written out by the
 * chain rule one query row at a time: the step that "FlashAttention and Fused
 * Kernels: Attention Without the n x n Matrix" ("Training: recompute instead
 * of store") and "Flash Attention, tiled" ("More arithmetic can still be
 * faster") describe as recomputing S and P from the inputs.  For query row i
 * with visible keys J_i and softmax row P_i:
 *     dP_ij = <dO_i, v_j>
 *     D_i   = sum_{j in J_i} P_ij dP_ij          (the softmax Jacobian term)
 *     dS_ij = P_ij (dP_ij - D_i)
 *     dQ_i  = scale * sum_j dS_ij k_j
 *     dK_j += scale * dS_ij q_i,   dV_j += P_ij dO_i
 * With grouped heads the contributions of every query head of a group add up
 * in its key/value head.
 *
 * row_pieces: P_ij (into p) and dS_ij (into ds) of one row; returns nothing.
 */
static void row_pieces(const double* qi, const double* doi, const double* kh, const double* vh,
                       int64_t n_vis, int64_t d, double scale, double* p, double* ds)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < n_vis; ++j) {
        const double* kj = kh + j * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += qi[c] * kj[c];
        p[j] = scale * dot;
        if (p[j] > m) m = p[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
    }
    for (int64_t j = 0; j < n_vis; ++j)
        p[j] /= l;
    double D = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        const double* vj = vh + j * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += doi[c] * vj[c];
        ds[j] = dot;                       /* dP_ij for now */
        D += p[j] * dot;
    }
    for (int64_t j = 0; j < n_vis; ++j)
        ds[j] = p[j] * (ds[j] - D);
}

int fa_ref_attn_bwd_f64(const double* q, const double* k, const double* v, const double* dout,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                        int causal, double scale,
                        double* dq, double* dk, double* dv)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
    if (!general_ok(B, Hq, Hkv, Tq, Tk, d, causal)) return -1;
    const int64_t group = Hq / Hkv;

    int failed = 0;
    /* One key/value head per iteration: it alone writes its dK and dV rows,
     * adding the rows of its query heads in a fixed order. */
#pragma omp parallel
    {
        double* p = (double*)malloc((size_t)Tk * sizeof(double));
        double* ds = (double*)malloc((size_t)Tk * sizeof(double));
        if (!p || !ds) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bkv = 0; bkv < B * Hkv; ++bkv) {
            if (!p || !ds) continue;
            const int64_t b = bkv / Hkv, hk = bkv % Hkv;
            const double* kh = k + bkv * Tk * d;
            const double* vh = v + bkv * Tk * d;
            double* dkh = dk + bkv * Tk * d;
            double* dvh = dv + bkv * Tk * d;
            for (int64_t x = 0; x < Tk * d; ++x) {
                dkh[x] = 0.0;
                dvh[x] = 0.0;
            }
            for (int64_t g = 0; g < group; ++g) {
                const int64_t bh = b * Hq + hk * group + g;
                for (int64_t i = 0; i < Tq; ++i) {
                    const int64_t flat = bh * Tq + i;
                    const double* qi = q + flat * d;
                    const double* doi = dout + flat * d;
                    double* dqi = dq + flat * d;
                    const int64_t n_vis = visible_of(flat, Tq, Tk, causal);
                    row_pieces(qi, doi, kh, vh, n_vis, d, scale, p, ds);
                    for (int64_t c = 0; c < d; ++c)
                        dqi[c] = 0.0;
                    for (int64_t j = 0; j < n_vis; ++j) {
                        const double* kj = kh + j * d;
                        for (int64_t c = 0; c < d; ++c) {
                            dqi[c] += scale * ds[j] * kj[c];
                            dkh[j * d + c] += scale * ds[j] * qi[c];
                            dvh[j * d + c] += p[j] * doi[c];
                        }
                    }
                }
            }
        }
        free(p);
        free(ds);
    }
    return failed ? -2 : 0;
}

/*
 * Selected gradient rows of the same backward: dQ for the flat query rows
 * qrows[r] = (b*Hq + h)*Tq + i, and dK, dV for the flat key rows
 * krows[r] = (b*Hkv + hk)*Tk + j.  A key row needs P_ij and D_i of every
 * query row that sees it, so the row statistics (log-sum-exp and D) of the
 * query heads of every listed key row are computed first, over all their
 * rows.  Same formulas as fa_ref_attn_bwd_f64.
 */
int fa_ref_attn_bwd_rows_f64(const double* q, const double* k, const double* v, const double* dout,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                             int causal, double scale,
                             const int64_t* qrows, int64_t n_qrows, double* dq_rows,
                             const int64_t* krows, int64_t n_krows, double* dk_rows, double* dv_rows)
{
    return fa_ref_attn_bwd_rows_given_d_f64(q, k, v, dout, B, Hq, Hkv, Tq, Tk, d, causal, scale, NULL,
                                            qrows, n_qrows, dq_rows, krows, n_krows, dk_rows, dv_rows);
}

/*
 * The same with the softmax Jacobian term D_i taken from `d_rows` (one value
 * per flat query row, [B][Hq][Tq]) instead of computed as sum_j P_ij dP_ij;
 * NULL means computed.  With D_i = dO_i . O_i for the exact O this is the same
 * result (D_i = dO_i . O_i is an identity); it lets a test measure what a
 * rounded O in that product alone changes.
 */
int fa_ref_attn_bwd_rows_given_d_f64(const double* q, const double* k, const double* v, const double* dout,
                                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                                     int causal, double scale, const double* d_rows,
                                     const int64_t* qrows, int64_t n_qrows, double* dq_rows,
                                     const int64_t* krows, int64_t n_krows, double* dk_rows, double* dv_rows)
{
    if (!q || !k || !v || !dout) return -1;
    if (!general_ok(B, Hq, Hkv, Tq, Tk, d, causal) || n_qrows < 0 || n_krows < 0) return -1;
    if (n_qrows > 0 && (!qrows || !dq_rows)) return -1;
    if (n_krows > 0 && (!krows || !dk_rows || !dv_rows)) return -1;
    for (int64_t r = 0; r < n_qrows; ++r)
        if (qrows[r] < 0 || qrows[r] >= B * Hq * Tq) return -1;
    for (int64_t r = 0; r < n_krows; ++r)
        if (krows[r] < 0 || krows[r] >= B * Hkv * Tk) return -1;
    const int64_t group = Hq / Hkv;

    /* Query heads whose statistics the key rows need. */
    const int64_t n_bh = B * Hq;
    char* need = (char*)calloc((size_t)n_bh, 1);
    double* lse = (double*)malloc((size_t)n_bh * (size_t)Tq * sizeof(double));
    double* D = (double*)malloc((size_t)n_bh * (size_t)Tq * sizeof(double));
    if (!need || !lse || !D) {
        free(need); free(lse); free(D);
        return -2;
    }
    for (int64_t r = 0; r < n_krows; ++r) {
        const int64_t bkv = krows[r] / Tk;
        const int64_t b = bkv / Hkv, hk = bkv % Hkv;
        for (int64_t g = 0; g < group; ++g)
            need[b * Hq + hk * group + g] = 1;
    }

    int failed = 0;
#pragma omp parallel
    {
        double* p = (double*)malloc((size_t)Tk * sizeof(double));
        double* ds = (double*)malloc((size_t)Tk * sizeof(double));
        if (!p || !ds) {
#pragma omp atomic write
            failed = 1;
        }
        /* dQ rows: independent. */
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_qrows; ++r) {
            if (!p || !ds) continue;
            const int64_t flat = qrows[r];
            const int64_t kvh = kv_head_of(flat, Hq, Hkv, Tq);
            const double* kh = k + kvh * Tk * d;
            const int64_t n_vis = visible_of(flat, Tq, Tk, causal);
            row_pieces(q + flat * d, dout + flat * d, kh, v + kvh * Tk * d, n_vis, d, scale, p, ds);
            if (d_rows) {
                /* ds holds P (dP - D) for the computed D; rebuild it with the given one. */
                for (int64_t j = 0; j < n_vis; ++j) {
                    double dot = 0.0;
                    for (int64_t c = 0; c < d; ++c)
                        dot += dout[flat * d + c] * v[kvh * Tk * d + j * d + c];
                    ds[j] = p[j] * (dot - d_rows[flat]);
                }
            }
            double* out = dq_rows + r * d;
            for (int64_t c = 0; c < d; ++c)
                out[c] = 0.0;
            for (int64_t j = 0; j < n_vis; ++j)
                for (int64_t c = 0; c < d; ++c)
                    out[c] += scale * ds[j] * kh[j * d + c];
        }
        /* Row statistics of the needed heads: lse_i = m_i + ln l_i and D_i. */
#pragma omp for schedule(dynamic, 16)
        for (int64_t flat = 0; flat < n_bh * Tq; ++flat) {
            if (!p || !ds || !need[flat / Tq]) continue;
            const int64_t kvh = kv_head_of(flat, Hq, Hkv, Tq);
            const double* kh = k + kvh * Tk * d;
            const double* vh = v + kvh * Tk * d;
            const int64_t n_vis = visible_of(flat, Tq, Tk, causal);
            const double* qi = q + flat * d;
            const double* doi = dout + flat * d;
            double m = -INFINITY;
            for (int64_t j = 0; j < n_vis; ++j) {
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    dot += qi[c] * kh[j * d + c];
                p[j] = scale * dot;
                if (p[j] > m) m = p[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < n_vis; ++j)
                l += exp(p[j] - m);
            const double lse_i = m + log(l);
            double Di = 0.0;
            for (int64_t j = 0; j < n_vis; ++j) {
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    dot += doi[c] * vh[j * d + c];
                Di += exp(p[j] - lse_i) * dot;
            }
            lse[flat] = lse_i;
            D[flat] = d_rows ? d_rows[flat] : Di;
        }
        /* dK, dV rows: sums over the query rows that see the key. */
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_krows; ++r) {
            const int64_t bkv = krows[r] / Tk, j = krows[r] % Tk;
            const int64_t b = bkv / Hkv, hk = bkv % Hkv;
            const double* kj = k + krows[r] * d;
            const double* vj = v + krows[r] * d;
            double* dkj = dk_rows + r * d;
            double* dvj = dv_rows + r * d;
            for (int64_t c = 0; c < d; ++c) {
                dkj[c] = 0.0;
                dvj[c] = 0.0;
            }
            for (int64_t g = 0; g < group; ++g) {
                const int64_t bh = b * Hq + hk * group + g;
                for (int64_t i = 0; i < Tq; ++i) {
                    const int64_t flat = bh * Tq + i;
                    if (j >= visible_of(flat, Tq, Tk, causal)) continue;
                    const double* qi = q + flat * d;
                    const double* doi = dout + flat * d;
                    double s = 0.0, dp = 0.0;
                    for (int64_t c = 0; c < d; ++c) {
                        s += qi[c] * kj[c];
                        dp += doi[c] * vj[c];
                    }
                    const double pij = exp(scale * s - lse[flat]);
                    const double dsij = pij * (dp - D[flat]);
                    for (int64_t c = 0; c < d; ++c) {
                        dkj[c] += scale * dsij * qi[c];
                        dvj[c] += pij * doi[c];
                    }
                }
            }
        }
        free(p);
        free(ds);
    }
    free(need); free(lse); free(D);
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
