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
    FA_ERR_HIP = 8,      /* the HIP launch itself failed                        */
    FA_ERR_SPLIT = 9,    /* num_splits outside 1 .. ceil(N / fa_tile_keys(d))   */
    FA_ERR_SCRATCH = 10  /* fa_fwd_splitkv_static: partials exceed its scratch  */
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
 *   H         heads, >= 1, with H * d <= 4194304.
 *   N         sequence length (dense) or total tokens T (packed), >= 1.
 *   d         head dimension: 64, 128 or 256.
 *   scale     softmax scale applied to Q K^T in fp32 (usually 1/sqrt(d)),
 *             finite and > 0.
 *   causal    0 or non-zero (lower-triangular mask).
 *   cu_seqlens NULL (dense) or a device int32 array of B+1 non-decreasing
 *             offsets with cu_seqlens[0] = 0 and cu_seqlens[B] = N.  Its
 *             contents are read on the device and not validated (no
 *             synchronisation); every kernel clamps sequence b to tokens
 *             [clamp(cu[b], 0, N), clamp(cu[b+1], that, N)), so malformed
 *             offsets give wrong results, never accesses outside the
 *             buffers.  This holds for every packed entry point.
 *   stream    HIP stream the kernel is queued on (NULL: default stream).
 * Returns FA_OK or an fa_status code.  Uses the library's default variant:
 * hardware exp2 and the strict conditional rescale (O and l are rescaled only
 * when some row's maximum grows; the largest weight of a row is then exactly 1
 * in bf16).  The threshold rule is faster on unit-variance inputs but lets a
 * dominant weight reach 2^8, which bf16 cannot hold exactly, so its instances
 * divide O by the sum of the bf16 weights at some cost (see fa_fwd_variant).
 * The workgroup shape follows the size of the grid (fa_fwd_tile_rows); the
 * results do not.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int N, int d, float scale, int causal,
           const int32_t *cu_seqlens, hipStream_t stream);

/*
 * fa_fwd_variant: fa_fwd with an explicit exp evaluation (fa_exp_mode) and
 * rescale policy (fa_rescale_mode).  Every variant computes the same O and
 * LSE up to rounding, within the forward's tolerances; they differ in speed.
 * Its workgroups always have fa_tile_rows(d) rows, so (FA_EXP_HW,
 * FA_RESCALE_STRICT) is fa_fwd with the tile it uses on large grids.
 * Threshold instances divide O by the sum of the bf16-rounded weights that
 * the P V product uses (its reference max may trail a row's maximum by up to
 * 8, so a dominant weight is not exact in bf16); the LSE always uses the fp32
 * sum.
 */
int fa_fwd_variant(const void *q, const void *k, const void *v, void *o,
                   float *lse, int B, int H, int N, int d, float scale,
                   int causal, const int32_t *cu_seqlens, hipStream_t stream,
                   int exp_mode, int rescale_mode);

/*
 * fa_fwd_pingpong: fa_fwd (hardware exp2, strict rescale) with another
 * schedule of the same arithmetic -- the ping-pong of two query tiles of
 * "Understanding FlashAttention V4", section 3.1: the two halves of each
 * eight-wave workgroup (one wave of each on every SIMD, 128 query rows each)
 * run half a key tile apart, separated by a barrier every half tile, so that
 * one half's load issue, rescale of O and barrier wait fall under the other
 * half's matrix products.  Head dimension 128 only (FA_ERR_HEAD_DIM for 64
 * and 256; other values as fa_fwd).  Outputs are bitwise fa_fwd's; every
 * other argument, the layouts and the errors are fa_fwd's.  Measured slower
 * than fa_fwd's schedule (both halves in step, each wave interleaving its
 * products with its softmax) on MI355X.
 */
int fa_fwd_pingpong(const void *q, const void *k, const void *v, void *o,
                    float *lse, int B, int H, int N, int d, float scale,
                    int causal, const int32_t *cu_seqlens, hipStream_t stream);

/*
 * Split-KV forward (dense layout; packed: fa_fwd_splitkv_packed).  For every (b, h) and query tile of
 * fa_tile_rows(d) rows, the keys that tile sees (all N, or when causal those
 * up to its last row) are cut into num_splits consecutive ranges of whole
 * K/V tiles of near-equal length: with T such tiles, range s holds tiles
 * [floor(s T / num_splits), floor((s + 1) T / num_splits)) (fa_split_range
 * gives the keys; a range is empty when T < num_splits).  Each (query tile,
 * key range) pair is a
 * workgroup of its own, so the launch has num_splits times more parallel
 * work than fa_fwd: the parallelisation along the key sequence that the
 * FlashAttention-2 section of "FlashAttention 1-4 explained" describes, for
 * shapes whose B * H * ceil(N / fa_tile_rows(d)) workgroups cannot fill the
 * GPU.  A first kernel writes, per key range, the attention of every query
 * row over that range alone; a second (fa_merge) combines them.
 *
 *   q, k, v, o, lse, B, H, N, d, scale, causal   as fa_fwd (dense layout).
 *   num_splits  1 .. ceil(N / fa_tile_keys(d)); fa_num_splits suggests one.
 *   o_part      device fp32 workspace, [num_splits, B, N, H, d]
 *               (num_splits * B * N * H * d floats, 16-byte aligned).
 *               On return (after the stream work) it holds each range's
 *               normalised partial output; 0 for rows that see no key of
 *               the range (causal).
 *   lse_part    device fp32 workspace, [num_splits, B, H, N]; each range's
 *               partial LSE, -inf for rows that see no key of the range.
 * The workspaces belong to the caller, like every other buffer, and must
 * not overlap any input, output or each other.  O and LSE equal fa_fwd's up
 * to rounding (the fp32 partials are rounded to bf16 only after the merge).
 * Uses hardware exp and the threshold rescale.
 */
int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o,
                   float *lse, int B, int H, int N, int d, float scale,
                   int causal, int num_splits, float *o_part, float *lse_part,
                   hipStream_t stream);

/*
 * fa_fwd_splitkv_packed: fa_fwd_splitkv over packed sequences (the packed
 * layout of fa_fwd: q, k, v, o [T, H, d], lse [H, T], cu_seqlens device int32
 * [B + 1]; variable-length sequences are a case of the tile scheduler in
 * section 3.4 of "Understanding FlashAttention V4").  Each sequence's query
 * tiles are cut into key ranges as fa_fwd_splitkv cuts a dense sequence of
 * its length (fa_split_range with N = that length): a short sequence's
 * ranges past its last key tile are empty.
 *   num_splits  1 .. ceil(T / fa_tile_keys(d)).
 *   o_part      device fp32 workspace [num_splits, T, H, d].
 *   lse_part    device fp32 workspace [num_splits, H, T].
 * Each sequence's O and LSE are bitwise those of fa_fwd_splitkv on that
 * sequence alone with min(num_splits, ceil(n / fa_tile_keys(d))) ranges.
 * Errors as fa_fwd_splitkv;
 * FA_ERR_NULLPTR for cu_seqlens == NULL.
 */
int fa_fwd_splitkv_packed(const void *q, const void *k, const void *v, void *o,
                          float *lse, const int32_t *cu_seqlens, int B, int H,
                          int T, int d, float scale, int causal,
                          int num_splits, float *o_part, float *lse_part,
                          hipStream_t stream);

/* Size of the static scratch of fa_fwd_splitkv_static, per GPU: 64 MiB. */
#define FA_STATIC_SCRATCH_BYTES (64u << 20)

/*
 * fa_fwd_splitkv_static: fa_fwd_splitkv for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split partials live in a static
 * device array of FA_STATIC_SCRATCH_BYTES that each GPU the library runs on
 * holds until the process ends (its address is looked up once per device,
 * on that device's first call, with the caller's device current); the call
 * itself allocates and frees nothing.
 *   Arguments as fa_fwd_splitkv without o_part / lse_part.  The partials
 *   take num_splits * B * N * H * (d + 1) * 4 bytes; more than
 *   FA_STATIC_SCRATCH_BYTES returns FA_ERR_SCRATCH before any HIP call.
 * Results are bitwise those of fa_fwd_splitkv (the same kernels).  Every
 * call on one GPU shares that GPU's scratch and leaves its partials there
 * (each call writes every partial it reads, so nothing needs clearing):
 * calls that overlap on one GPU -- on different streams, or from several
 * threads -- race, and the caller must order them.
 */
int fa_fwd_splitkv_static(const void *q, const void *k, const void *v,
                          void *o, float *lse, int B, int H, int N, int d,
                          float scale, int causal, int num_splits,
                          hipStream_t stream);

/*
 * fa_merge: the combination step of fa_fwd_splitkv, usable on its own (for
 * example on partials computed over key shards held elsewhere).  For each
 * row, with LSE_s and O_s the partials of range s,
 *     LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s,
 * which is exact because each O_s is a softmax-weighted mean over its own
 * keys.  A row whose partials are all empty (LSE_s = -inf) gets O = 0 and
 * LSE = -inf.
 *   o_part, lse_part  device fp32 partials, layouts as in fa_fwd_splitkv.
 *   o, lse            device outputs: bf16 [B, N, H, d], fp32 [B, H, N].
 * Errors as fa_fwd (FA_ERR_SPLIT for num_splits < 1).
 */
int fa_merge(const float *o_part, const float *lse_part, int num_splits,
             int B, int H, int N, int d, void *o, float *lse,
             hipStream_t stream);

/* Keys [*key_lo, *key_hi) of range s of fa_fwd_splitkv for query row `row`
 * (the range of its query tile; the row itself, when causal, sees only the
 * keys <= row of it).  Returns FA_OK, FA_ERR_NULLPTR, FA_ERR_SHAPE (N < 1 or
 * row outside [0, N)), FA_ERR_HEAD_DIM or FA_ERR_SPLIT (num_splits or s out
 * of range). */
int fa_split_range(int N, int d, int causal, int num_splits, int s, int row,
                   int *key_lo, int *key_hi);

/* A split count for fa_fwd_splitkv on a GPU with num_cus compute units
 * (<= 0: 256).  Returns 1 (use fa_fwd) when fa_fwd's workgroups (counted
 * half when causal) already fill every resident slot (3, 1 or 1 workgroups
 * per compute unit at d = 64, 128, 256), or fill one per compute unit and
 * N < 8192; otherwise enough ranges to fill the slots, each at least 1024
 * keys long, at most 32. */
int fa_num_splits(int B, int H, int N, int d, int causal, int num_cus);

/*
 * fa_bwd: gradients of exact attention (d = 64, 128 or 256), dense or packed.
 * For the forward O = softmax(scale Q K^T) V and an upstream gradient dO it
 * writes
 *     dV = P^T dO,  dQ = scale dS K,  dK = scale dS^T Q,
 *     dS = P * (dP - delta),  dP = dO V^T,  delta_i = sum_d dO_id O_id,
 * with P recomputed from the forward's log-sum-exp instead of being stored
 * (the recomputation of the FlashAttention-1 backward in the summary table
 * of "FlashAttention 1-4 explained").  No atomics are used: results are
 * bitwise reproducible run to run (the deterministic mode of section 3.3 of
 * "Understanding FlashAttention V4").
 *   q, k, v, o, dout  device bf16, the forward's layout: [B, N, H, d], or
 *                     [T, H, d] with cu_seqlens: the forward's inputs, its
 *                     output O and the upstream gradient dO.
 *   lse               device fp32, the forward's LSE: [B, H, N] or [H, T].
 *   dq, dk, dv        device bf16 outputs in the layout of q.
 *   cu_seqlens        as fa_fwd: NULL (dense) or device int32 [B + 1]
 *                     sequence offsets, N = T; each sequence is its own
 *                     attention problem.
 *   workspace         device fp32 scratch of two floats per LSE entry,
 *                     fa_bwd_workspace_floats(B, H, N) dense and
 *                     fa_bwd_workspace_floats(1, H, T) packed (16-byte
 *                     aligned); overwritten.
 *   B, H, N, scale, causal, stream   as fa_fwd.
 * Three kernels are queued on `stream`.  Outputs and the workspace must not
 * overlap any input or each other.  Errors as fa_fwd.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o,
           const float *lse, const void *dout, void *dq, void *dk, void *dv,
           int B, int H, int N, int d, float scale, int causal,
           const int32_t *cu_seqlens, float *workspace, hipStream_t stream);

/* Size of fa_bwd's workspace in floats: 2 * B * H * N (0 for an invalid
 * shape); for packed sequences pass B = 1 and N = T. */
long long fa_bwd_workspace_floats(int B, int H, int N);

/*
 * fa_fwd_rescale_counts: fa_fwd_variant (hardware exp2, d = 128 only) in an
 * instance that also counts how often the conditional rescale of the online
 * softmax ("FlashAttention 1-4 explained", FlashAttention-4 section: rescale
 * only when the maximum grows; "Understanding FlashAttention V4", section 3.2:
 * only when overflow is possible) actually rescales.  It writes O and LSE like
 * fa_fwd_variant and ADDS to four device counters (the caller zeroes them):
 *   counts[0]  wave-steps after each wave's first key tile (one per 64-key
 *              tile and 32-row wave),
 *   counts[1]  of those, steps whose O accumulator was rescaled (some row of
 *              the wave moved its reference max),
 *   counts[2]  rows whose reference max moved, over the same tiles,
 *   counts[3]  rows updated (32 per counted wave-step).
 * The atomics make it slower than fa_fwd: a measurement tool, not a variant.
 *   rescale_mode  FA_RESCALE_STRICT or FA_RESCALE_THRESHOLD
 *   counts        device array of 4 unsigned 64-bit integers, 8-byte aligned,
 *                 not overlapping q, k, v, o or lse; borrowed.
 * Returns fa_fwd_variant's codes, FA_ERR_NULLPTR for counts == NULL,
 * FA_ERR_ALIGN, FA_ERR_HEAD_DIM for d != 128, FA_ERR_VARIANT for another
 * rescale_mode, FA_ERR_ALIAS for overlapping counters.
 */
int fa_fwd_rescale_counts(const void *q, const void *k, const void *v, void *o,
                          float *lse, int B, int H, int N, int d, float scale,
                          int causal, const int32_t *cu_seqlens,
                          hipStream_t stream, int rescale_mode,
                          unsigned long long *counts);

/*
 * fa_fwd_masked: fa_fwd with a window mask and an optional linear distance
 * bias (dense layout) -- built-in forms of the score modifications and masks
 * that FlexAttention user code expresses (FlashAttention-4 as a FlexAttention
 * backend: "FlashAttention 1-4 explained", FlashAttention-4 section).
 *   window_left, window_right   key j is visible to query i iff
 *                  i - window_left <= j <= i + window_right; a negative value
 *                  leaves that side unbounded (window_right = 0 with an
 *                  unbounded left side is the causal mask); an edge of N - 1
 *                  or more hides no key and is taken as N - 1 (so INT_MAX
 *                  also means unbounded).  Key tiles that no row of a
 *                  workgroup sees are skipped.
 *   alibi_slopes   NULL, or device fp32 [H]: slope_h * (j - i) is added to
 *                  the scaled score (ALiBi).
 * Every other argument as fa_fwd (no cu_seqlens, no causal flag); N is at
 * most 2^30 (FA_ERR_SHAPE beyond).  Uses hardware exp and the threshold
 * rescale; tiles that a window edge cuts and the sequence tail go through the
 * mask step, and with a bias every other tile adds the bias alone.
 */
int fa_fwd_masked(const void *q, const void *k, const void *v, void *o,
                  float *lse, int B, int H, int N, int d, float scale,
                  int window_left, int window_right, const float *alibi_slopes,
                  hipStream_t stream);

/*
 * fa_fwd_masked_packed: fa_fwd_masked over packed sequences (q, k, v, o
 * [T, H, d], lse [H, T], cu_seqlens device int32 [B + 1] as fa_fwd).  Row
 * and key positions i, j count from each sequence's first token, and a
 * query sees only its own sequence's keys; the window and the bias are
 * otherwise as fa_fwd_masked's.  T <= 2^30.  Errors as fa_fwd_masked;
 * FA_ERR_NULLPTR for cu_seqlens == NULL.
 */
int fa_fwd_masked_packed(const void *q, const void *k, const void *v, void *o,
                         float *lse, const int32_t *cu_seqlens, int B, int H,
                         int T, int d, float scale, int window_left,
                         int window_right, const float *alibi_slopes,
                         hipStream_t stream);

/*
 * FP8 forward (dense layout, d = 64, 128 or 256).  The FlashAttention-3 notes of
 * "FlashAttention 1-4 explained" run the forward's products on FP8 matrix
 * units; here Q K^T and P V both run on E4M3 operands (OCP E4M3: bias 7,
 * largest finite 448, 0x7f/0xff NaN) with fp32 accumulation.  Scaling is per
 * (b, h): a tensor's real values are code * descale[b * H + h].
 *   q8, k8     device E4M3 codes [B, N, H, d].
 *   vt8        device E4M3 codes of V transposed, [B, H, d, Np] with
 *              Np = fa_fp8_vt_stride(N) = ceil(N / 64) * 64; the padding
 *              columns must hold finite codes (fa_quantize_fp8 writes 0).
 *   descale_q, descale_k, descale_v   device fp32 [B * H].
 *   o, lse     device outputs: bf16 [B, N, H, d], fp32 [B, H, N].
 *   B, H, N, scale, causal, stream    as fa_fwd.
 * P = exp(s - m) is rounded to E4M3 after scaling by 2^8 (P <= 1: the
 * running max is exact, strict rescale), so each weight carries a relative
 * rounding error of at most 2^-4; the row sum and LSE come from the fp32 P.
 */
int fa_fwd_fp8(const void *q8, const void *k8, const void *vt8,
               const float *descale_q, const float *descale_k,
               const float *descale_v, void *o, float *lse, int B, int H,
               int N, int d, float scale, int causal, hipStream_t stream);

/*
 * fa_quantize_fp8: per-(b, h) E4M3 quantisation of a bf16 tensor x
 * [B, N, H, d] (d = 64, 128 or 256): descale[b * H + h] = amax / 448 over
 * that head (1 for an all-zero head) and codes = E4M3(x * (1 / descale)),
 * rounded to nearest even, every step in fp32.  transpose = 0 writes x8 as
 * [B, N, H, d]; transpose != 0 writes [B, H, d, fa_fp8_vt_stride(N)] with
 * zero codes in the padding (the V layout of fa_fwd_fp8).  Four kernels on
 * `stream`: until the last one, descale holds each head's running amax (so
 * it must not alias x or x8); the amax is reduced over 256-token slices and
 * merged with an atomic maximum, which is exact, so the result does not
 * depend on the order of the workgroups.  Errors as fa_fwd.
 */
int fa_quantize_fp8(const void *x, void *x8, float *descale, int B, int H,
                    int N, int d, int transpose, hipStream_t stream);

/* Row stride (keys) of the transposed FP8 V layout: ceil(N / 64) * 64. */
int fa_fp8_vt_stride(int N);

/*
 * Packed sequences in FP8 ("Understanding FlashAttention V4", section 3.4,
 * names variable-length sequences as a case of the tile scheduler): B
 * sequences in T tokens, cu_seqlens as fa_fwd's (device int32 [B + 1],
 * cu_seqlens[0] = 0, non-decreasing, cu_seqlens[B] = T; read on the device,
 * not validated, clamped as fa_fwd's; a sequence whose padded keys would end
 * past the V^T row, which only malformed offsets such as overlapping
 * sequences produce, is skipped).  Each sequence is its own attention
 * problem with its own per-head scales.
 *
 * fa_fp8_vt_stride_packed: row length (keys) of the packed transposed V
 * layout [H, d, Tp]: Tp = ceil(T / 64) * 64 + 64 B, which holds every
 * sequence's keys padded to a multiple of 64; 0 for T < 1, B < 1 or a
 * length past 2^31 - 1.  Sequence b's keys start at column
 * sum_{b' < b} ceil(n_b' / 64) * 64.
 */
int fa_fp8_vt_stride_packed(int T, int B);

/*
 * fa_quantize_fp8_packed: fa_quantize_fp8 per (sequence, head) of a packed
 * bf16 x [T, H, d]: descale[b * H + h] = amax / 448 over sequence b's tokens
 * of head h (1 when all zero or the sequence is empty).  transpose = 0
 * writes x8 as [T, H, d]; transpose != 0 writes the packed V^T layout
 * [H, d, fa_fp8_vt_stride_packed(T, B)]: sequence b's codes and zero codes up
 * to its next multiple of 64 keys; the columns past the last sequence's
 * padding are not written.  The same four kernels on `stream`, each
 * sequence's tokens cut into equal slices for the amax and the codes.
 * Errors as fa_quantize_fp8; FA_ERR_NULLPTR for cu_seqlens == NULL.
 */
int fa_quantize_fp8_packed(const void *x, void *x8, float *descale,
                           const int32_t *cu_seqlens, int B, int H, int T,
                           int d, int transpose, hipStream_t stream);

/*
 * fa_fwd_fp8_packed: fa_fwd_fp8 over packed sequences.
 *   q8, k8     device E4M3 codes [T, H, d].
 *   vt8        device E4M3 codes in the packed V^T layout
 *              [H, d, fa_fp8_vt_stride_packed(T, B)]; each sequence's padding
 *              columns must hold finite codes (fa_quantize_fp8_packed writes 0).
 *   descale_q, descale_k, descale_v   device fp32 [B * H] per (sequence, head).
 *   o, lse     device outputs: bf16 [T, H, d], fp32 [H, T].
 *   cu_seqlens, B, T   as above; H, d, scale, causal, stream as fa_fwd_fp8.
 * Work items are (sequence, head, query tile) decoded from cu_seqlens like
 * the packed fa_fwd.  Errors as fa_fwd_fp8; FA_ERR_NULLPTR for
 * cu_seqlens == NULL.
 */
int fa_fwd_fp8_packed(const void *q8, const void *k8, const void *vt8,
                      const float *descale_q, const float *descale_k,
                      const float *descale_v, void *o, float *lse,
                      const int32_t *cu_seqlens, int B, int H, int T, int d,
                      float scale, int causal, hipStream_t stream);

/* Static, NUL-terminated description of an fa_status code. */
const char *fa_strerror(int code);

/* Rows per workgroup tile and keys per K/V tile at head dimension d (0 for
 * an unsupported d): the query tile of the split-KV, masked, counting,
 * ping-pong and fa_fwd_variant instances, and of fa_fwd on grids that fill
 * the GPU (fa_fwd_tile_rows gives fa_fwd's choice for a shape).
 * Informational; no result depends on it. */
int fa_tile_rows(int d);
int fa_tile_keys(int d);

/* Rows per workgroup tile that fa_fwd (hardware exp2, strict rescale) uses
 * for a shape on a GPU with num_cus compute units (<= 0: 256, the MI355X);
 * fa_fwd itself asks HIP for the current device's count once per device.
 * B, N: batch and sequence length (packed: the sequence count and T).  At
 * d = 128 the grid of 256-row eight-wave workgroups is replaced by 128-row
 * four-wave ones when the former would leave compute units idle: with
 * items = ceil(N / 256) * B * H (packed: * H alone), non-causal when items is
 * at most num_cus / 2, or strictly between num_cus and 3 num_cus with
 * items mod num_cus in 1 .. num_cus / 2 (a last round at most half full);
 * causal when items is at most 1.5 num_cus.  Each query row sees the same key
 * tiles in the same order either way, so O and LSE are bitwise the same
 * (finite inputs).  Other d: their fixed tile.  0 for an unsupported d;
 * fa_tile_rows(d) for B, H or N < 1.  Informational, like fa_tile_rows. */
int fa_fwd_tile_rows(int B, int H, int N, int d, int causal, int packed, int num_cus);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
