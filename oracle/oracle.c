/*
 * Exact scaled-dot-product attention, forward pass, in fp64 -- the oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * CPU definition that the fused HIP kernel is checked against.  Only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark may load
 * it; the product path never does.  It shares no code, header or table with
 * the GPU path.
 *
 * What it computes (FlashAttention explainer pages: "1.1 the self-attention
 * compute chain", and the "standard attention" equation block of the
 * "FlashAttention 1-4 explained" post):
 *
 *     S = Q K^T * scale          (scores, one full row at a time)
 *     m = max_j S_ij             (row max, subtracted for stability)
 *     P_ij = exp(S_ij - m) / sum_j exp(S_ij - m)
 *     O = P V
 *
 * plus the per-row log-sum-exp LSE_i = m_i + ln(sum_j exp(S_ij - m_i)), which
 * the pages do not define: it is the natural-log normaliser of the scaled
 * scores, the quantity a backward pass would reuse.
 *
 * Reading of the pages used here (they are silent on all of these):
 *   - inputs are bf16 bit patterns, widened exactly to double;
 *   - scale is the fp32 value the GPU receives, widened to double;
 *   - causal keeps key j for query i iff j <= i (the lower triangle the
 *     FlashAttention-2 engineering notes skip to);
 *   - dense tensors are [B, N, H, d]; packed variable-length tensors are
 *     [T, H, d] with sequence b spanning tokens cu_seqlens[b]..cu_seqlens[b+1].
 *
 * A key range [kv_lo, kv_hi) may further restrict the visible keys.  The
 * result is then the attention of each row over that part of the sequence
 * alone: the partial output and log-sum-exp that a split of the key/value
 * sequence produces (the "parallel along the sequence" discussion of the
 * FlashAttention 1-4 post, FlashAttention-2 section).  A row that sees no
 * key in the range gets O = 0 and LSE = -inf, the neutral element of the
 * merge that combines such partials.
 *
 * The S row is materialised in full, exactly as the naive method of the
 * pages does (and as the fused kernel avoids); memory stays bounded because
 * only one row per thread exists at a time.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_OK = 0, ORACLE_ERR_ARG = 1, ORACLE_ERR_ROW = 2, ORACLE_ERR_ALLOC = 3 };

static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

struct job {
    const uint16_t *q, *k, *v;
    int B, H, N, d, causal;
    int kv_lo, kv_hi;           /* key range, intersected with the visible keys */
    double scale;
    const int32_t *cu;          /* NULL for dense */
    const int64_t *rows;        /* triples (b, h, i) */
    int64_t first, last;        /* this thread's share of rows */
    double *o, *lse;
    int status;
};

/* Start token and length of sequence b. */
static void seq_span(const struct job *jb, int b, int64_t *start, int *len)
{
    if (jb->cu) {
        *start = jb->cu[b];
        *len = jb->cu[b + 1] - jb->cu[b];
    } else {
        *start = (int64_t)b * jb->N;
        *len = jb->N;
    }
}

static void one_row(const struct job *jb, int64_t r, double *s)
{
    const int b = (int)jb->rows[3 * r], h = (int)jb->rows[3 * r + 1];
    const int i = (int)jb->rows[3 * r + 2];
    const int d = jb->d, H = jb->H;
    int64_t t0;
    int n;
    seq_span(jb, b, &t0, &n);

    /* visible keys: j < n, and j <= i when causal; then [kv_lo, kv_hi) */
    const int nvis = jb->causal ? i + 1 : n;
    const int lo = jb->kv_lo > 0 ? jb->kv_lo : 0;
    const int hi = jb->kv_hi < nvis ? jb->kv_hi : nvis;
    const uint16_t *qi = jb->q + ((t0 + i) * H + h) * (int64_t)d;
    double *oi = jb->o + r * (int64_t)d;
    if (hi <= lo) {
        /* no key: empty sum, O = 0 and LSE = ln 0 */
        for (int x = 0; x < d; ++x) oi[x] = 0.0;
        jb->lse[r] = -INFINITY;
        return;
    }

    /* S_ij = scale * (q_i . k_j).  Each dot product is the plain sum over
     * x = 0 .. d-1 in order; KB keys are summed side by side only so that
     * the additions of different keys overlap in the CPU (every S_ij is
     * bit-for-bit what the one-key-at-a-time loop gives). */
    enum { KB = 8 };
    double *qd = s + jb->N;     /* q_i widened once (the row buffer holds N + d) */
    for (int x = 0; x < d; ++x) qd[x] = widen_bf16(qi[x]);
    int j = lo;
    for (; j + KB <= hi; j += KB) {
        const uint16_t *kj[KB];
        double dot[KB];
        for (int u = 0; u < KB; ++u) {
            kj[u] = jb->k + ((t0 + j + u) * H + h) * (int64_t)d;
            dot[u] = 0.0;
        }
        for (int x = 0; x < d; ++x)
            for (int u = 0; u < KB; ++u)
                dot[u] += qd[x] * widen_bf16(kj[u][x]);
        for (int u = 0; u < KB; ++u) s[j + u] = jb->scale * dot[u];
    }
    for (; j < hi; ++j) {
        const uint16_t *kj = jb->k + ((t0 + j) * H + h) * (int64_t)d;
        double dot = 0.0;
        for (int x = 0; x < d; ++x)
            dot += qd[x] * widen_bf16(kj[x]);
        s[j] = jb->scale * dot;
    }

    /* m = row max; e_j = exp(S_ij - m); l = sum e_j */
    double m = -INFINITY;
    for (int j = lo; j < hi; ++j)
        if (s[j] > m) m = s[j];
    double l = 0.0;
    for (int j = lo; j < hi; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }

    /* O_i = sum_j (e_j / l) v_j */
    for (int x = 0; x < d; ++x) oi[x] = 0.0;
    for (int j = lo; j < hi; ++j) {
        const double p = s[j] / l;
        const uint16_t *vj = jb->v + ((t0 + j) * H + h) * (int64_t)d;
        for (int x = 0; x < d; ++x)
            oi[x] += p * widen_bf16(vj[x]);
    }
    jb->lse[r] = m + log(l);
}

static void *worker(void *arg)
{
    struct job *jb = (struct job *)arg;
    /* one score row (N) and the widened query row (d) */
    double *s = (double *)malloc(sizeof(double) * ((size_t)(jb->N > 0 ? jb->N : 1) + (size_t)jb->d));
    if (!s) {
        jb->status = ORACLE_ERR_ALLOC;
        return NULL;
    }
    for (int64_t r = jb->first; r < jb->last; ++r)
        one_row(jb, r, s);
    free(s);
    return NULL;
}

/*
 * Attention output for a list of rows, over the keys j in [kv_lo, kv_hi)
 * that the row sees.
 *   q, k, v   host bf16 bit patterns, [B, N, H, d] (cu_seqlens == NULL) or
 *             [T, H, d] (cu_seqlens != NULL, T = cu_seqlens[B]).
 *   N         sequence length (dense) or the longest sequence (packed); it
 *             sizes the per-thread score row.
 *   rows      n_rows triples (b, h, i): sequence, head, query index within
 *             the sequence.
 *   kv_lo, kv_hi  key range (indices within the sequence); 0 and N for all.
 *   o_out     n_rows x d doubles; lse_out n_rows doubles.
 *   nthreads  worker threads (>= 1).
 * Returns 0, or a non-zero code for a bad argument or row.
 */
int oracle_attention_rows_range(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                int B, int H, int N, int d, float scale, int causal,
                                const int32_t *cu_seqlens, int64_t n_rows,
                                const int64_t *rows, int kv_lo, int kv_hi,
                                double *o_out, double *lse_out, int nthreads)
{
    if (!q || !k || !v || !rows || !o_out || !lse_out) return ORACLE_ERR_ARG;
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || n_rows < 0 || nthreads <= 0)
        return ORACLE_ERR_ARG;

    struct job base;
    memset(&base, 0, sizeof base);
    base.q = q; base.k = k; base.v = v;
    base.B = B; base.H = H; base.N = N; base.d = d; base.causal = causal != 0;
    base.kv_lo = kv_lo; base.kv_hi = kv_hi;
    base.scale = (double)scale;
    base.cu = cu_seqlens;
    base.rows = rows;
    base.o = o_out; base.lse = lse_out;

    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || i < 0) return ORACLE_ERR_ROW;
        int64_t t0;
        int n;
        seq_span(&base, (int)b, &t0, &n);
        if (i >= n || n > N) return ORACLE_ERR_ROW;
    }

    if (nthreads > n_rows) nthreads = n_rows > 0 ? (int)n_rows : 1;
    struct job *jobs = (struct job *)calloc((size_t)nthreads, sizeof *jobs);
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof *tid);
    char *joinable = (char *)calloc((size_t)nthreads, 1);
    if (!jobs || !tid || !joinable) {
        free(jobs);
        free(tid);
        free(joinable);
        return ORACLE_ERR_ALLOC;
    }
    int rc = ORACLE_OK;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].first = n_rows * t / nthreads;
        jobs[t].last = n_rows * (t + 1) / nthreads;
        if (pthread_create(&tid[t], NULL, worker, &jobs[t]) == 0)
            joinable[t] = 1;
        else
            worker(&jobs[t]); /* no thread available: run the share here */
    }
    for (int t = 0; t < nthreads; ++t) {
        if (joinable[t]) pthread_join(tid[t], NULL);
        if (jobs[t].status != ORACLE_OK) rc = jobs[t].status;
    }
    free(jobs);
    free(tid);
    free(joinable);
    return rc;
}

/* Attention output for a list of rows over every visible key (see above). */
int oracle_attention_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          int B, int H, int N, int d, float scale, int causal,
                          const int32_t *cu_seqlens, int64_t n_rows,
                          const int64_t *rows, double *o_out, double *lse_out,
                          int nthreads)
{
    return oracle_attention_rows_range(q, k, v, B, H, N, d, scale, causal, cu_seqlens,
                                       n_rows, rows, 0, N, o_out, lse_out, nthreads);
}
