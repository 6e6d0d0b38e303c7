/*
 * fa.h -- C ABI of the exact attention forward and backward for MI355X (gfx950).
 *
 * The exact attention forward of one or more heads:
 *
 *   O[b,h,i,:] = sum_{j visible to i} softmax_j(scale * q_i . k_j) * v_j
 *   lse[b,h,i] = ln sum_{j visible to i} exp(scale * q_i . k_j)
 *
 * with "visible" meaning every key j < T, or, when causal, every key j <= i.
 * The problem statement -- (B, H, T, d) tensors, the score matrix scaled by
 * 1/sqrt(d) by default, future keys masked to -inf before the softmax -- is
 * the one given on "Flash Attention, tiled: exact attention without the T x T
 * HBM matrix", section "Ordinary causal attention".  The computation is the
 * tiled online-softmax forward of the same page ("From the example to tiled
 * GPU work") and of "FlashAttention: the IO-aware Attention Kernel",
 * sections 3.2-3.3: the T x T score and probability matrices never reach
 * memory.  The per-row log-sum-exp is the extra per-row scalar of
 * "FlashAttention and Fused Kernels: Attention Without the n x n Matrix",
 * Step 4, returned in natural-log units, so that P_ij = exp(s_ij - lse_i).
 *
 * fa_bwd is its training backward (the gradients with respect to q, k, v).
 * All entry points are plain C: pointers, sizes and a HIP stream handle.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,      /* a required pointer is NULL                          */
    FA_ERR_SHAPE = 2,     /* a size < 1, Hq not a multiple of Hkv, or causal with
                             Tq > Tk                                             */
    FA_ERR_HEAD_DIM = 3,  /* d is not 64 or 128                                  */
    FA_ERR_SCALE = 4,     /* scale is NaN or infinite, or scale * log2(e)
                             overflows fp32 (|scale| > ~2.36e38)                */
    FA_ERR_ALIGN = 5,     /* q, k, v, o not 16-byte aligned, or lse not 4-byte   */
    FA_ERR_OVERFLOW = 6,  /* sizes overflow 64-bit byte counts or the launch grid,
                             or one head (T*d*2 bytes plus 2 row tiles) >= 4 GiB */
    FA_ERR_HIP = 7,       /* the kernel launch failed; see fa_hip_error_string()  */
    FA_ERR_ARG = 8,       /* causal not 0/1, n_split < 1, workspace too small, or
                             overlapping buffers                                 */
    FA_ERR_SCRATCH = 9    /* fa_fwd_split_noalloc: the split needs more than
                             FA_SCRATCH_BYTES of scratch                         */
} fa_status;

/* Size of the library's fixed split-key scratch (fa_fwd_split_noalloc). */
#define FA_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * fa_fwd -- exact attention forward, enqueued on `stream`.
 *
 * q, k, v : device pointers to bf16 tensors of shape [B][H][T][d], dense
 *           row-major (d fastest), 16-byte aligned.  Read only.
 * o       : device pointer, bf16 [B][H][T][d], same layout; written with
 *           round-to-nearest-even from the fp32 result.
 * lse     : device pointer, fp32 [B][H][T]; natural-log log-sum-exp of the
 *           visible scaled scores of each row.
 * B, H, T : batch, heads, sequence length (queries and keys alike), >= 1.
 * d       : head size, 64 or 128.
 * causal  : 1 = key j visible to query i iff j <= i; 0 = every key visible.
 * scale   : multiplies q.k; any finite value with |scale| <= ~2.36e38, so
 *           that scale * log2(e) is finite in fp32 (callers usually pass
 *           1/sqrt(d)); 0 gives uniform weights.  The exponent arithmetic
 *           is fp32: a row whose largest visible scaled score, in log2 units
 *           |scale * q.k * log2(e)|, reaches 2^23 (~8.4e6) has no accurate
 *           result (far past where the softmax is a hard maximum), and its o
 *           and lse are written as NaN, never as a plausible-looking value.
 * stream  : HIP stream to enqueue on; NULL means the default stream.
 *
 * Ownership: the caller allocates and owns every buffer.  The library
 * allocates no memory, keeps no per-call state and is reentrant; o and lse
 * must not overlap q, k or v.
 *
 * Errors: every argument is validated before any HIP call.  On a validation
 * failure nothing is launched and the matching FA_ERR_* code is returned.
 * FA_ERR_HIP means the launch was rejected by the runtime; the message is
 * available from fa_hip_error_string() on the same thread.  FA_OK means the
 * work was enqueued; completion is observed by synchronising the stream.
 * Unsupported shapes are rejected, never redirected to another algorithm.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v,
                 void* o, float* lse,
                 int64_t B, int64_t H, int64_t T, int64_t d,
                 int causal, float scale, hipStream_t stream);

/*
 * fa_fwd_gqa -- fa_fwd with grouped key/value heads.
 *
 * Llama 3.1 8B shares each key/value head among four query heads
 * ("FlashAttention and Fused Kernels: Attention Without the n x n Matrix",
 * Step 4).  Here q and o are [B][Hq][T][d], k and v are [B][Hkv][T][d], and
 * query head h reads key/value head h / (Hq / Hkv): consecutive query heads
 * share one.  Hq must be a multiple of Hkv (else FA_ERR_SHAPE); Hkv == Hq is
 * fa_fwd.  Everything else (layout, lse, ownership, errors) is as for fa_fwd.
 */
fa_status fa_fwd_gqa(const void* q, const void* k, const void* v,
                     void* o, float* lse,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t d,
                     int causal, float scale, hipStream_t stream);

/*
 * fa_fwd_split -- the general forward, with the keys split across workgroups.
 *
 * This is Flash-Decoding ("FlashAttention and Fused Kernels: Attention Without
 * the n x n Matrix", Step 4).  The keys are cut into n_split contiguous
 * chunks of whole 64-key tiles, each chunk is attended by its own
 * workgroups, and a second kernel merges the chunks with the log-sum-exp
 * combine of the same step.  This gives a short query block (decode: Tq = 1)
 * against a long cache enough parallel work.
 *
 * q, o    : bf16 [B][Hq][Tq][d];  k, v : bf16 [B][Hkv][Tk][d];  lse : fp32
 *           [B][Hq][Tq].  Hq a multiple of Hkv; head mapping as fa_fwd_gqa.
 * causal  : the query rows are the last Tq positions of the Tk-long sequence,
 *           so query i sees keys j <= i + (Tk - Tq).  This needs Tq <= Tk
 *           (else FA_ERR_SHAPE).  Without causal, Tq and Tk are free.
 * n_split : >= 1.  Chunks are ceil(Tk / n_split) keys, rounded up to a
 *           multiple of 64, so fewer chunks than asked may exist.  When one
 *           chunk results, no workspace is used and no combine runs.
 * workspace, workspace_bytes : device scratch owned by the caller, 16-byte
 *           aligned, at least fa_fwd_split_workspace_bytes(...) bytes.  It holds
 *           each chunk's fp32 output and log-sum-exp.  It may be NULL when
 *           that size is 0; it must not overlap any other buffer.
 *
 * Grouped heads with no mask (or one query row per head) run as one problem
 * per key/value head with Hq / Hkv * Tq query rows, so every key/value tile is
 * read once per group rather than once per query head.
 *
 * A row is written as NaN (o and lse) as for fa_fwd, and also when the
 * largest visible scaled score of any one of its chunks reaches 2^23 in log2
 * units: each chunk's partial result is held to the same fp32 range.
 *
 * The workspace is overwritten on every call; calls that share it must not
 * run concurrently.  The two kernels are enqueued in order on `stream`.
 * Errors as fa_fwd, plus: FA_ERR_NULL for a missing workspace, and
 * FA_ERR_ARG for n_split < 1, a workspace that is too small, or overlaps.
 */
fa_status fa_fwd_split(const void* q, const void* k, const void* v,
                       void* o, float* lse,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                       int causal, float scale, int64_t n_split,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_fwd_split_noalloc -- fa_fwd_split for callers that cannot allocate.
 *
 * For code that may not call hipMalloc: under HIP graph capture, inside tight
 * serving loops, or in harnesses that forbid allocation.  It runs exactly
 * fa_fwd_split's kernels (same results, bit for bit), but the chunks' partial
 * results go to a fixed scratch buffer inside the library instead of a caller
 * workspace.  The arguments are fa_fwd_split's without the workspace.
 *
 * Scratch: FA_SCRATCH_BYTES (16 MiB) of device memory per GPU, a static array
 * that each GPU the library runs on holds until the process ends.  A call
 * needs fa_fwd_split_workspace_bytes(B, Hq, Tq, Tk, d, n_split) bytes of it;
 * a larger need returns FA_ERR_SCRATCH before any HIP call (for example,
 * d = 128 with n_split = 8 fits 4064 query rows).  The first call on a device
 * looks up the array's device address once (hipGetSymbolAddress); no call
 * allocates or frees memory.  The scratch needs no clearing: every chunk
 * writes all of its rows before the combine reads them.
 *
 * Every call on a GPU shares that GPU's scratch and leaves it holding its
 * partials: calls that overlap on one GPU (several streams or host threads)
 * race and give wrong results.  Serialise them.  The stream's device
 * selects the scratch; the calling thread's current device is unchanged.
 * Errors as fa_fwd_split (no workspace errors), plus FA_ERR_SCRATCH.
 */
fa_status fa_fwd_split_noalloc(const void* q, const void* k, const void* v,
                               void* o, float* lse,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk,
                               int64_t d, int causal, float scale, int64_t n_split,
                               hipStream_t stream);

/* Workspace bytes fa_fwd_split needs for these sizes (0: none needed, or
 * invalid sizes). */
size_t fa_fwd_split_workspace_bytes(int64_t B, int64_t Hq, int64_t Tq, int64_t Tk, int64_t d,
                                    int64_t n_split);

/* A split count that gives the GPU enough workgroups for these sizes (1
 * when the query tiles alone fill it).  Advice only; any n_split >= 1 is
 * valid. */
int64_t fa_fwd_split_count(int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d, int causal);

/*
 * fa_fwd_fp8 -- the forward with FP8 E4M3 inputs, enqueued on `stream`.
 *
 * The FP8 mode named for FlashAttention-3 ("FlashAttention and Fused Kernels:
 * Attention Without the n x n Matrix", "Four generations"; the pages give no
 * recipe).  The operands are descale * e4m3: q, k, v hold OCP FP8 E4M3 bytes
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; the patterns
 * 0x7F / 0xFF are NaN and must not occur) with one fp32 descale factor per
 * tensor, and the result is the attention of those values:
 *
 *   O[b,h,i,:] = sum_j softmax_j(scale * qd * kd * q_i . k_j) * vd * v_j
 *
 * with the head mapping and causal rule of fa_fwd_split (no key split).  Both
 * products run on the FP8 matrix cores; the probability weights enter the PV
 * product rounded to E4M3 (round to nearest even), the only approximation
 * beyond rounding order.  The weights are 2^3 * exp2 of the score against a
 * lazily moved reference that never exceeds the row max; they lie in
 * (0, 448] and the largest is at least 8.  O is normalised by the sum of the
 * rounded weights, so each output element is within
 *   sum_j max(2^-4 w_j, min(2^-13 / Z, w_j)) |vd v_j - O| (to first order)
 * of the exact value, w the exact weights and Z = sum_j exp(s_j - max s),
 * plus the matrix cores' summation of each 64-product block (measured within
 * 2^-10.9 of the largest product), fp32 accumulation and the bf16 store.
 * lse uses fp32 weights.
 *
 * q       : device pointer, E4M3 bytes [B][Hq][Tq][d], 16-byte aligned.
 * k, v    : device pointers, E4M3 bytes [B][Hkv][Tk][d], 16-byte aligned.
 * o       : device pointer, bf16 [B][Hq][Tq][d], 16-byte aligned.
 * lse     : device pointer, fp32 [B][Hq][Tq], natural log, 4-byte aligned.
 * B, Hq, Hkv, Tq, Tk, d, causal, scale : as fa_fwd_split.
 * q_descale, k_descale, v_descale : finite and > 0 (else FA_ERR_SCALE);
 *           scale * q_descale * k_descale * log2(e) must be finite in fp32.
 * stream  : HIP stream; NULL means the default stream.
 *
 * Ownership, validation and errors as fa_fwd: nothing is allocated, o and
 * lse must not overlap the inputs (FA_ERR_ARG), FA_ERR_HIP carries the
 * runtime's message in fa_hip_error_string().
 */
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v,
                     void* o, float* lse,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                     int causal, float scale, float q_descale, float k_descale, float v_descale,
                     hipStream_t stream);

/*
 * fa_fwd_fp8_split -- fa_fwd_fp8 with the keys split across workgroups.
 *
 * Flash-Decoding ("FlashAttention and Fused Kernels: Attention Without the
 * n x n Matrix", Step 4) over FP8 E4M3 inputs: the keys are cut into n_split
 * chunks exactly as for fa_fwd_split, each chunk's workgroups write their
 * normalised fp32 output and log-sum-exp into the workspace, and the same
 * log-sum-exp combine merges them into o and lse.  A decode step against an
 * E4M3 cache reads half the bytes of a bf16 one.
 *
 * Arguments as fa_fwd_fp8, plus n_split, workspace and workspace_bytes as
 * fa_fwd_split; the workspace layout and size are those of fa_fwd_split
 * (fa_fwd_split_workspace_bytes gives the size, fa_fwd_split_count advice
 * on n_split).  n_split = 1, or any n_split that leaves one chunk, is
 * fa_fwd_fp8 and uses no workspace.  Errors as fa_fwd_fp8, plus FA_ERR_NULL
 * for a missing workspace and FA_ERR_ARG for n_split < 1, a workspace that is
 * too small, or overlaps.  The workspace is overwritten on every call; calls
 * that share it must not run concurrently.
 */
fa_status fa_fwd_fp8_split(const void* q, const void* k, const void* v,
                           void* o, float* lse,
                           int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                           int causal, float scale, float q_descale, float k_descale, float v_descale,
                           int64_t n_split, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_bwd -- gradients of the exact attention forward, enqueued on `stream`.
 *
 * The backward that keeps only O and the per-row log-sum-exp from the forward
 * and recomputes the score and probability tiles from q and k ("FlashAttention
 * and Fused Kernels: Attention Without the n x n Matrix", "Training: recompute
 * instead of store").  With P_ij = exp(scale * q_i . k_j - lse_i) over the
 * visible keys, dP = dO V^T, D_i = dO_i . O_i and dS = P * (dP - D):
 *     dq = scale * dS K,   dk = scale * dS^T Q,   dv = P^T dO,
 * where dk and dv of a key/value head add up every query head of its group.
 *
 * q, o, dout, dq : bf16 [B][Hq][Tq][d];  k, v, dk, dv : bf16 [B][Hkv][Tk][d];
 *           dense row-major, 16-byte aligned.  o and lse are what the forward
 *           (fa_fwd, fa_fwd_gqa or fa_fwd_split) returned for these q, k, v,
 *           causal and scale; dout is the upstream gradient of o.
 * lse     : fp32 [B][Hq][Tq], natural-log units, 4-byte aligned, finite.
 * dq, dk, dv : written (bf16, round-to-nearest-even from fp32 sums); they must
 *           not overlap each other, any input or the workspace.
 * B, Hq, Hkv, Tq, Tk, d, causal, scale : as fa_fwd_split (head mapping, causal
 *           rule for the last Tq positions, Tq <= Tk when causal).
 * workspace, workspace_bytes : device scratch owned by the caller, 16-byte
 *           aligned, at least fa_bwd_workspace_bytes(B, Hq, Tq) bytes; it
 *           holds D and lse * log2(e) per row and is overwritten.  Calls that
 *           share it must not run concurrently.
 *
 * Three kernels are enqueued in order: the per-row D, then dk and dv, then
 * dq.  No atomics are used: equal inputs give bit-equal gradients.
 * Errors as fa_fwd_split; FA_ERR_NULL if any pointer (workspace included) is
 * NULL, FA_ERR_ARG for a workspace that is too small or overlapping buffers.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv,
                 int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int64_t d,
                 int causal, float scale, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes fa_bwd needs: 8 per query row (0 for invalid sizes). */
size_t fa_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Tq);

/* Static, human-readable text for a status code (never NULL).  status is an
 * fa_status value; any other int gives "unknown status". */
const char* fa_status_string(int status);

/* Text of the HIP error of the calling thread's last call of any entry point
 * above, or "" when that call launched successfully */
const char* fa_hip_error_string(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
