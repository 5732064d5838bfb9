/*
 * fa.h -- C ABI of the fused exact-attention forward for AMD Instinct MI355X
 * (gfx950 / CDNA4).  Library: libfa.so.
 *
 * The operation is the forward pass of exact scaled-dot-product attention,
 *
 *     O = softmax(Q K^T * scale) V,
 *
 * as defined by the compute chain of section 1.1 of "Understanding
 * FlashAttention V4" (scores, subtract the row max, exp and normalise, P V)
 * and by the "standard attention" equation block of "FlashAttention 1-4
 * explained".  It is computed as one fused, tiled kernel with the online
 * softmax of the FlashAttention-1 derivation in that post: S and P never
 * reach HBM; per row only the running max, the running sum and the
 * unnormalised output are carried, and the division by the sum happens once
 * at the end (the FlashAttention-2 deferred normalisation).
 *
 * Besides O the call writes the per-row log-sum-exp of the scaled scores,
 *     LSE_i = ln sum_{visible j} exp(scale * q_i . k_j),
 * in natural-log units (the pages do not define it; it is what a backward
 * pass would reuse).
 *
 * Layouts (all tensors contiguous, row-major):
 *   dense  (cu_seqlens == NULL): q, k, v, o are [B, N, H, d] bf16;
 *                                lse is [B, H, N] fp32.
 *   packed (cu_seqlens != NULL): B sequences of lengths
 *          n_b = cu_seqlens[b+1] - cu_seqlens[b] packed along one token axis
 *          of T = cu_seqlens[B] tokens; q, k, v, o are [T, H, d] bf16 and lse
 *          is [H, T] fp32.  N must equal T.  Queries and keys of a sequence
 *          have the same length; a packed call with one sequence is
 *          byte-identical to the dense call with B = 1.
 * bf16 values are raw 16-bit patterns (IEEE binary32 upper half).
 *
 * causal != 0 keeps key j for query i iff j <= i (positions local to each
 * sequence): the lower triangle, whose fully masked tiles the kernel never
 * visits (FlashAttention-2 engineering notes).
 *
 * Ownership and synchronisation: every buffer belongs to the caller and must
 * be device memory on the current device, stay alive until the work queued
 * on `stream` has finished, and not overlap `o` or `lse` with any input.  The
 * library allocates nothing, keeps no pointer after returning, never
 * synchronises and holds no global state, so calls are thread-safe.
 * `stream` is borrowed; NULL means the default stream.
 *
 * Errors: arguments are validated before anything is enqueued; on a non-zero
 * return nothing was launched and no output was touched.  Faults inside the
 * kernel (for example a malformed cu_seqlens array, whose contents the host
 * cannot see) surface at the caller's next synchronisation of `stream`.
 */
#ifndef FA_H
#define FA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

enum fa_status {
    FA_OK = 0,
    FA_ERR_NULLPTR = 1,  /* q, k, v, o or lse is NULL                          */
    FA_ERR_SHAPE = 2,    /* B, H or N < 1, sizes overflow, or grid too large   */
    FA_ERR_HEAD_DIM = 3, /* d is not 64, 128 or 256                            */
    FA_ERR_SCALE = 4,    /* scale is not finite or not > 0                      */
    FA_ERR_ALIGN = 5,    /* q, k, v, o not 16-byte aligned, lse or cu_seqlens
                            not 4-byte aligned                                  */
    FA_ERR_VARIANT = 6,  /* exp_mode or rescale_mode out of range               */
    FA_ERR_ALIAS = 7,    /* o or lse overlaps an input or each other            */
    FA_ERR_HIP = 8       /* the HIP launch itself failed                        */
};

/* How P~ = exp(s - m) is evaluated (section 3.2 of the FlashAttention V4
 * explainer moves exp from the special-function unit to FMA units). */
enum fa_exp_mode {
    FA_EXP_HW = 0,    /* hardware v_exp_f32 (native 2^x)                        */
    FA_EXP_POLY = 1,  /* degree-3 minimax polynomial for 2^f on FMA units       */
    FA_EXP_MIXED = 2  /* half of each row's exps on each unit                   */
};

/* When the running output and sum are rescaled by exp(m_old - m_new)
 * (conditional rescale: FlashAttention-4 section of "FlashAttention 1-4
 * explained", and section 3.2 of the V4 explainer).  All three are exact:
 * the output and the sum always share one reference max. */
enum fa_rescale_mode {
    FA_RESCALE_ALWAYS = 0,    /* every tile                                     */
    FA_RESCALE_STRICT = 1,    /* skipped by a wave when no row max grew         */
    FA_RESCALE_THRESHOLD = 2  /* the reference max moves only when a row max
                                 exceeds it by more than 8 (log2 units), so
                                 that P~ stays <= 2^8                            */
};

/*
 * fa_fwd: O and LSE of exact attention (see the file comment).
 *   q, k, v   device bf16 inputs (layout above), read only.
 *   o         device bf16 output, same shape as q.
 *   lse       device fp32 output, [B, H, N] (dense) or [H, T] (packed).
 *   B         batch size (dense) or number of packed sequences, >= 1.
 *   H         heads, >= 1.
 *   N         sequence length (dense) or total tokens T (packed), >= 1.
 *   d         head dimension: 64, 128 or 256.
 *   scale     softmax scale applied to Q K^T in fp32 (usually 1/sqrt(d)),
 *             finite and > 0.
 *   causal    0 or non-zero (lower-triangular mask).
 *   cu_seqlens NULL (dense) or a device int32 array of B+1 non-decreasing
 *             offsets with cu_seqlens[0] = 0 and cu_seqlens[B] = N.
 *   stream    HIP stream the kernel is queued on (NULL: default stream).
 * Returns FA_OK or an fa_status code.  Uses the library's default variant
 * (hardware exp, strict conditional rescale).
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int N, int d, float scale, int causal,
           const int32_t *cu_seqlens, hipStream_t stream);

/*
 * fa_fwd_variant: fa_fwd with an explicit exp evaluation (fa_exp_mode) and
 * rescale policy (fa_rescale_mode).  Every variant computes the same O and
 * LSE up to rounding; they differ only in speed.
 */
int fa_fwd_variant(const void *q, const void *k, const void *v, void *o,
                   float *lse, int B, int H, int N, int d, float scale,
                   int causal, const int32_t *cu_seqlens, hipStream_t stream,
                   int exp_mode, int rescale_mode);

/* Static, NUL-terminated description of an fa_status code. */
const char *fa_strerror(int code);

/* Rows per workgroup tile and keys per K/V tile of the kernel that fa_fwd
 * would launch for head dimension d (0 for an unsupported d).  Informational;
 * used by benchmarks to report launch geometry. */
int fa_tile_rows(int d);
int fa_tile_keys(int d);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
