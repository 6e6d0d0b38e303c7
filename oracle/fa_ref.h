/*
 * fa_ref.h -- CPU oracle for the exact attention forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this.  It is used by the tests, by the smoke check and by the
 * benchmark's CPU-baseline leg, and by nothing else.  It shares no code,
 * header, table or helper with the GPU library.
 *
 * What it computes (one row at a time, no tiling, everything in double):
 *
 *   For every batch b, head h and query row i, with J_i the visible keys
 *   (all j < T, or j <= i when causal):
 *     s_ij  = scale * sum_k q[b,h,i,k] * k[b,h,j,k]          for j in J_i
 *     m_i   = max_{j in J_i} s_ij
 *     l_i   = sum_{j in J_i} exp(s_ij - m_i)
 *     O_i   = sum_{j in J_i} exp(s_ij - m_i) * v[b,h,j,:] / l_i
 *     lse_i = m_i + ln(l_i)
 *
 * Sources: the score matrix, the (B, H, T, d) naming and the causal rule
 * (key j visible to query i iff j <= i, masked scores become -inf before
 * the softmax) are from "Flash Attention, tiled: exact attention without
 * the T x T HBM matrix", section "Ordinary causal attention".  Subtracting
 * the row maximum before exponentiating is from the same page, section
 * "What happens when the maximum changes", and from "FlashAttention and
 * Fused Kernels: Attention Without the n x n Matrix", Step 2.  The
 * per-row log-sum-exp is the extra scalar per row named in the same
 * vidyal.ai page, Step 4 ("Flash-Decoding: split the cache, not the
 * queries"), read as the natural log of the row's softmax denominator
 * including the max shift.
 *
 * Layout: q, k, v are dense row-major [B][H][T][d] arrays of double; o is
 * [B][H][T][d] double; lse is [B][H][T] double.  The caller owns every
 * buffer.  Return value: 0 on success, -1 on invalid sizes or NULL
 * pointers, -2 if a scratch allocation fails.
 */
#ifndef FA_REF_H
#define FA_REF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every row of every (b, h). */
int fa_ref_fwd_f64(const double* q, const double* k, const double* v,
                   double* o, double* lse,
                   int64_t B, int64_t H, int64_t T, int64_t d,
                   int causal, double scale);

/* Only the listed rows.  rows[r] is a flat row index (b*H + h)*T + i.
 * o_rows is [n_rows][d], lse_rows is [n_rows]; q, k, v as above. */
int fa_ref_fwd_rows_f64(const double* q, const double* k, const double* v,
                        int64_t B, int64_t H, int64_t T, int64_t d,
                        int causal, double scale,
                        const int64_t* rows, int64_t n_rows,
                        double* o_rows, double* lse_rows);

/* The general problem: q, o are [B][Hq][Tq][d], k, v are [B][Hkv][Tk][d];
 * query head h reads key/value head h / (Hq / Hkv); with causal, query i sees
 * keys j <= i + (Tk - Tq) (the queries are the last Tq positions).  Needs
 * Hq % Hkv == 0, and Tq <= Tk when causal.  lse is [B][Hq][Tq]. */
int fa_ref_attn_f64(const double* q, const double* k, const double* v,
                    double* o, double* lse,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                    int causal, double scale);

/* Selected rows of the general problem; rows[r] = (b*Hq + h)*Tq + i. */
int fa_ref_attn_rows_f64(const double* q, const double* k, const double* v,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                         int causal, double scale,
                         const int64_t* rows, int64_t n_rows,
                         double* o_rows, double* lse_rows);

/* Backward of the general problem for upstream gradient dout ([B][Hq][Tq][d]):
 * dq is [B][Hq][Tq][d], dk and dv are [B][Hkv][Tk][d] (each the sum over the
 * query heads of its group).  With P the softmax rows, dP = dout V^T,
 * D_i = sum_j P_ij dP_ij and dS = P * (dP - D): dq = scale dS K,
 * dk = scale dS^T Q, dv = P^T dout.  Same return codes as above. */
int fa_ref_attn_bwd_f64(const double* q, const double* k, const double* v, const double* dout,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                        int causal, double scale,
                        double* dq, double* dk, double* dv);

/* Selected rows of the backward: dq for flat query rows qrows[r] =
 * (b*Hq + h)*Tq + i into dq_rows [n_qrows][d]; dk, dv for flat key rows
 * krows[r] = (b*Hkv + hk)*Tk + j into dk_rows, dv_rows [n_krows][d]. */
int fa_ref_attn_bwd_rows_f64(const double* q, const double* k, const double* v, const double* dout,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                             int causal, double scale,
                             const int64_t* qrows, int64_t n_qrows, double* dq_rows,
                             const int64_t* krows, int64_t n_krows, double* dk_rows, double* dv_rows);

/* fa_ref_attn_bwd_rows_f64 with the softmax Jacobian term D_i of every flat
 * query row given in d_rows ([B][Hq][Tq]) instead of computed; NULL means
 * computed, exactly as fa_ref_attn_bwd_rows_f64. */
int fa_ref_attn_bwd_rows_given_d_f64(const double* q, const double* k, const double* v, const double* dout,
                                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                                     int causal, double scale, const double* d_rows,
                                     const int64_t* qrows, int64_t n_qrows, double* dq_rows,
                                     const int64_t* krows, int64_t n_krows, double* dk_rows, double* dv_rows);

/* Number of OpenMP threads the oracle runs with. */
int fa_ref_num_threads(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_REF_H */
