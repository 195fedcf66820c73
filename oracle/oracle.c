/*
 * oracle.c -- plain fp64 CPU reference for one layer of Orthros phase-aware
 * heterogeneous attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load or call this file's library.  The
 * GPU library never links it and shares no code, header or table with it.
 *
 * Pages cited (by title and section):
 *   [N]  "Orthros:阶段感知异构注意力精读笔记" (close-reading notes of
 *        arXiv 2610.13735).
 *
 * What is computed, in the pages' order:
 *   - per-stream query scale-offset: q_hat = q * alpha + beta for the base
 *     stream and q_hat' = q' * alpha' + beta' for the output-only stream,
 *     from one shared projection ([N] §2.2, the symbol table; the display
 *     formula itself did not survive, this is the reading the symbol table
 *     gives: alpha, beta are 1 x d vectors applied elementwise);
 *   - base stream: causal sliding-window attention over the window
 *     W_t = {max(1, t-w+1), ..., t} ([N] §2.3, Eq. (4)), for every base
 *     position;
 *   - the base stream writes every position's K/V into the layer's cache;
 *     the window bounds reads, not storage ([N] §2.1, §2.6);
 *   - output-only stream: full-history causal cross-attention over the
 *     cache, keys j <= t where t is the copy's ORIGINAL position, not its
 *     slot ([N] §2.3 Eq. (5), §2.4);
 *   - prefill: one copy per sequence; decode: one base token and one copy
 *     per step, the copy reading the whole history including the new token
 *     ([N] §2.4 walk-through, §2.5 mode table);
 *   - pre-training and fine-tuning modes: T_out copies per sequence at
 *     arbitrary original positions (every position in PT, the answer
 *     positions in SFT; [N] §2.5 mode table), each the Eq. (5) query of its
 *     own position.
 *
 * Positions are 0-based here: the window of row t is [max(0, t-w+1), t].
 * Softmax uses the textbook max-subtracted form in fp64.  Every input is
 * read from its storage type (fp32, or bf16 as raw 16-bit patterns) and
 * promoted exactly to double.  Cache slots are written as byte copies of
 * the input rows, in the input's storage type.
 *
 * Layouts (row-major, contiguous):
 *   q, o            [B][T][Hq][d]      q_out, o_out  [B][Hq][d]
 *   k, v            [B][T][Hkv][d]     alpha..beta'  [Hq][d]
 *   k_cache,v_cache [B][Hkv][cap][d]
 * Query head h reads KV head h / (Hq/Hkv).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t batch, n_q_heads, n_kv_heads, head_dim, window;
    int32_t dtype;    /* 0: fp32 storage, 1: bf16 storage (uint16 bits) */
    int32_t nthreads; /* worker threads; <= 0 means 1 */
    double softmax_scale;
} oracle_shape;

/* Exact promotion of element i of a tensor stored as fp32 or bf16. */
static double ld(const void* p, int dtype, int64_t i)
{
    if (dtype == 0) return (double)((const float*)p)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static size_t elem_size(int dtype) { return dtype == 0 ? 4 : 2; }

/*
 * Softmax attention of one query over the keys lo..hi (inclusive) of one KV
 * head: z_j = scale * <qh, k_j>, o = sum_j exp(z_j - max z) v_j / sum_j
 * exp(z_j - max z).  Key j's row starts at element (base + j * stride) of
 * kbuf and vbuf.  This is the common form of [N] §2.3 Eqs. (4) and (5); the
 * two equations differ only in the key set.
 */
static void attend(const double* qh, int d, double scale,
                   const void* kbuf, const void* vbuf, int dtype,
                   int64_t base, int64_t stride, int64_t lo, int64_t hi,
                   double* out)
{
    int64_t n = hi - lo + 1;
    double* z = (double*)malloc((size_t)n * sizeof(double));
    double zmax = -INFINITY;
    for (int64_t j = lo; j <= hi; ++j) {
        int64_t row = base + j * stride;
        double dot = 0.0;
        for (int i = 0; i < d; ++i) dot += qh[i] * ld(kbuf, dtype, row + i);
        z[j - lo] = scale * dot;
        if (z[j - lo] > zmax) zmax = z[j - lo];
    }
    double denom = 0.0;
    for (int i = 0; i < d; ++i) out[i] = 0.0;
    for (int64_t j = lo; j <= hi; ++j) {
        double e = exp(z[j - lo] - zmax);
        denom += e;
        int64_t row = base + j * stride;
        for (int i = 0; i < d; ++i) out[i] += e * ld(vbuf, dtype, row + i);
    }
    for (int i = 0; i < d; ++i) out[i] /= denom;
    free(z);
}

/* q_hat = q * alpha + beta for query head h ([N] §2.2, symbol table). */
static void scale_offset(const void* q, int64_t qrow, const void* alpha,
                         const void* beta, int h, int d, int dtype, double* qh)
{
    for (int i = 0; i < d; ++i)
        qh[i] = ld(q, dtype, qrow + i) * ld(alpha, dtype, (int64_t)h * d + i)
              + ld(beta, dtype, (int64_t)h * d + i);
}

/* ---------------------------------------------------------------- threads */

typedef void (*unit_fn)(void* ctx, int64_t unit);
typedef struct { unit_fn fn; void* ctx; int64_t n_units; int tid, nthreads; } worker_arg;

static void* worker(void* p)
{
    worker_arg* a = (worker_arg*)p;
    for (int64_t u = a->tid; u < a->n_units; u += a->nthreads) a->fn(a->ctx, u);
    return NULL;
}

/* Runs fn(ctx, u) for u in [0, n_units), units dealt round-robin to threads. */
static void parallel_for(int nthreads, int64_t n_units, unit_fn fn, void* ctx)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    worker_arg args[256];
    for (int t = 0; t < nthreads; ++t) {
        args[t].fn = fn; args[t].ctx = ctx; args[t].n_units = n_units;
        args[t].tid = t; args[t].nthreads = nthreads;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, worker, &args[t]);
    worker(&args[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------- prefill */

typedef struct {
    const oracle_shape* s;
    int64_t T, cap;
    const void *q, *q_out, *k, *v, *alpha, *beta, *alpha_out, *beta_out;
    const int64_t* out_pos;
    const void *k_cache, *v_cache;
    double *o, *o_out;
} prefill_ctx;

/* Unit = (b, h): Eq. (4) for every base row t of head h of sequence b. */
static void prefill_swa_unit(void* p, int64_t u)
{
    prefill_ctx* c = (prefill_ctx*)p;
    const oracle_shape* s = c->s;
    int Hq = s->n_q_heads, Hkv = s->n_kv_heads, d = s->head_dim;
    int64_t b = u / Hq;
    int h = (int)(u % Hq), g = h / (Hq / Hkv);
    double* qh = (double*)malloc((size_t)d * sizeof(double));
    for (int64_t t = 0; t < c->T; ++t) {
        int64_t qrow = ((b * c->T + t) * Hq + h) * d;
        scale_offset(c->q, qrow, c->alpha, c->beta, h, d, s->dtype, qh);
        int64_t lo = t - s->window + 1;
        if (lo < 0) lo = 0;
        /* keys come from this layer's own K/V: row (b, j, g) */
        attend(qh, d, s->softmax_scale, c->k, c->v, s->dtype,
               (b * c->T * Hkv + g) * d, (int64_t)Hkv * d, lo, t,
               c->o + qrow);
    }
    free(qh);
}

/* Unit = (b, h): Eq. (5) for the one output copy of sequence b, keys
 * [0, out_pos[b]] of the cache ([N] §2.4: mask by original position). */
static void prefill_global_unit(void* p, int64_t u)
{
    prefill_ctx* c = (prefill_ctx*)p;
    const oracle_shape* s = c->s;
    int Hq = s->n_q_heads, Hkv = s->n_kv_heads, d = s->head_dim;
    int64_t b = u / Hq;
    int h = (int)(u % Hq), g = h / (Hq / Hkv);
    double* qh = (double*)malloc((size_t)d * sizeof(double));
    scale_offset(c->q_out, (b * Hq + h) * d, c->alpha_out, c->beta_out, h, d,
                 s->dtype, qh);
    attend(qh, d, s->softmax_scale, c->k_cache, c->v_cache, s->dtype,
           (b * Hkv + g) * c->cap * d, d, 0, c->out_pos[b],
           c->o_out + (b * Hq + h) * d);
    free(qh);
}

/*
 * One prefill call: cache write for positions [0, T), Eq. (4) for every
 * base row (skipped when o is NULL), Eq. (5) for one copy per sequence at
 * original position out_pos[b] (skipped when o_out is NULL).
 * Returns 0, or -1 on a bad shape or position.
 */
int oracle_prefill(const oracle_shape* s, int64_t T,
                   const void* q, const void* q_out, const int64_t* out_pos,
                   const void* k, const void* v,
                   const void* alpha, const void* beta,
                   const void* alpha_out, const void* beta_out,
                   void* k_cache, void* v_cache, int64_t cap,
                   double* o, double* o_out)
{
    if (!s || s->n_kv_heads < 1 || s->n_q_heads % s->n_kv_heads || s->window < 1 ||
        T < 1 || cap < T || (o_out && !out_pos))
        return -1;
    for (int b = 0; b < s->batch; ++b)
        if (out_pos && (out_pos[b] < 0 || out_pos[b] >= T)) return -1;
    int Hq = s->n_q_heads, Hkv = s->n_kv_heads, d = s->head_dim;
    size_t es = elem_size(s->dtype), row = (size_t)d * es;

    /* The base stream's K/V of every position go to the cache ([N] §2.1). */
    for (int64_t b = 0; b < s->batch; ++b)
        for (int g = 0; g < Hkv; ++g)
            for (int64_t j = 0; j < T; ++j) {
                size_t src = (size_t)(((b * T + j) * Hkv + g) * d) * es;
                size_t dst = (size_t)(((b * Hkv + g) * cap + j) * d) * es;
                memcpy((char*)k_cache + dst, (const char*)k + src, row);
                memcpy((char*)v_cache + dst, (const char*)v + src, row);
            }

    prefill_ctx c = {s, T, cap, q, q_out, k, v, alpha, beta, alpha_out, beta_out,
                     out_pos, k_cache, v_cache, o, o_out};
    int64_t units = (int64_t)s->batch * Hq;
    if (o) parallel_for(s->nthreads, units, prefill_swa_unit, &c);
    if (o_out) parallel_for(s->nthreads, units, prefill_global_unit, &c);
    return 0;
}

/* ---------------------------------------------------------- many copies */

typedef struct {
    const oracle_shape* s;
    int64_t T_out, cap;
    const void *q_out, *alpha_out, *beta_out, *k_cache, *v_cache;
    const int32_t* pos;
    double* o_out;
} copies_ctx;

/* Unit = (b, i, h): Eq. (5) for copy i of sequence b, query head h, keys
 * [0, pos[b][i]] of the cache. */
static void copies_unit(void* p, int64_t u)
{
    copies_ctx* c = (copies_ctx*)p;
    const oracle_shape* s = c->s;
    int Hq = s->n_q_heads, Hkv = s->n_kv_heads, d = s->head_dim;
    int h = (int)(u % Hq), g = h / (Hq / Hkv);
    int64_t bi = u / Hq, b = bi / c->T_out;
    int64_t qrow = (bi * Hq + h) * d;
    double* qh = (double*)malloc((size_t)d * sizeof(double));
    scale_offset(c->q_out, qrow, c->alpha_out, c->beta_out, h, d, s->dtype, qh);
    attend(qh, d, s->softmax_scale, c->k_cache, c->v_cache, s->dtype,
           (b * Hkv + g) * c->cap * d, d, 0, c->pos[bi], c->o_out + qrow);
    free(qh);
}

/*
 * Eq. (5) for T_out output copies per sequence ([N] §2.5 mode table: PT
 * copies every position, SFT the answer positions): copy i of sequence b
 * sits at original position pos[b][i] and attends the cached keys
 * [0, pos[b][i]] with its own query q_out[b][i] ([N] §2.4: the mask follows
 * the original position, never the copy's slot).  The copies neither write
 * the cache nor see one another.  Returns 0, or -1 on a bad shape or a
 * position outside [0, T).
 * Layouts: q_out, o_out [B][T_out][Hq][d], pos [B][T_out] (int32).
 */
int oracle_copies(const oracle_shape* s, int64_t T, int64_t T_out,
                  const void* q_out, const int32_t* pos,
                  const void* alpha_out, const void* beta_out,
                  const void* k_cache, const void* v_cache, int64_t cap,
                  double* o_out)
{
    if (!s || s->n_kv_heads < 1 || s->n_q_heads % s->n_kv_heads || T < 1 ||
        T_out < 1 || cap < T || !pos || !o_out)
        return -1;
    for (int64_t i = 0; i < (int64_t)s->batch * T_out; ++i)
        if (pos[i] < 0 || pos[i] >= T) return -1;
    copies_ctx c = {s, T_out, cap, q_out, alpha_out, beta_out, k_cache, v_cache,
                    pos, o_out};
    parallel_for(s->nthreads, (int64_t)s->batch * T_out * s->n_q_heads,
                 copies_unit, &c);
    return 0;
}

/* ---------------------------------------------------- sampled SWA rows */

typedef struct {
    const oracle_shape* s;
    int64_t T;
    const void *q, *k, *v, *alpha, *beta;
    const int64_t* rows;
    double* out;
} rows_ctx;

static void rows_unit(void* p, int64_t u)
{
    rows_ctx* c = (rows_ctx*)p;
    const oracle_shape* s = c->s;
    int Hq = s->n_q_heads, Hkv = s->n_kv_heads, d = s->head_dim;
    int64_t b = c->rows[3 * u], t = c->rows[3 * u + 1];
    int h = (int)c->rows[3 * u + 2], g = h / (Hq / Hkv);
    double qh[512];
    scale_offset(c->q, ((b * c->T + t) * Hq + h) * d, c->alpha, c->beta, h, d,
                 s->dtype, qh);
    int64_t lo = t - s->window + 1;
    if (lo < 0) lo = 0;
    attend(qh, d, s->softmax_scale, c->k, c->v, s->dtype,
           (b * c->T * Hkv + g) * d, (int64_t)Hkv * d, lo, t, c->out + u * d);
}

/*
 * Eq. (4) for a list of (b, t, h) rows only (rows holds n_rows triples);
 * out is [n_rows][d].  Used where the full prefill is too large for the
 * CPU.  Returns -1 on a row out of range or head_dim > 512.
 */
int oracle_swa_rows(const oracle_shape* s, int64_t T, const void* q,
                    const void* k, const void* v, const void* alpha,
                    const void* beta, int64_t n_rows, const int64_t* rows,
                    double* out)
{
    if (!s || s->head_dim > 512 || s->n_kv_heads < 1 ||
        s->n_q_heads % s->n_kv_heads || s->window < 1)
        return -1;
    for (int64_t u = 0; u < n_rows; ++u)
        if (rows[3 * u] < 0 || rows[3 * u] >= s->batch || rows[3 * u + 1] < 0 ||
            rows[3 * u + 1] >= T || rows[3 * u + 2] < 0 || rows[3 * u + 2] >= s->n_q_heads)
            return -1;
    rows_ctx c = {s, T, q, k, v, alpha, beta, rows, out};
    parallel_for(s->nthreads, n_rows, rows_unit, &c);
    return 0;
}

/* Unit = listed row u whose raw query is qrows[u] (not read from a full q). */
static void rows_given_q_unit(void* p, int64_t u)
{
    rows_ctx* c = (rows_ctx*)p;
    const oracle_shape* s = c->s;
    int Hq = s->n_q_heads, Hkv = s->n_kv_heads, d = s->head_dim;
    int64_t b = c->rows[3 * u], t = c->rows[3 * u + 1];
    int h = (int)c->rows[3 * u + 2], g = h / (Hq / Hkv);
    double qh[512];
    scale_offset(c->q, u * d, c->alpha, c->beta, h, d, s->dtype, qh);
    int64_t lo = t - s->window + 1;
    if (lo < 0) lo = 0;
    attend(qh, d, s->softmax_scale, c->k, c->v, s->dtype,
           (b * c->T * Hkv + g) * d, (int64_t)Hkv * d, lo, t, c->out + u * d);
}

/*
 * Eq. (4) for a list of (b, t, h) rows whose raw queries are passed row by
 * row (qrows [n_rows][d], in the storage type) instead of as a full
 * [B][T][Hq][d] tensor; k, v and the result as in oracle_swa_rows.  The
 * arithmetic is that of oracle_swa_rows, row for row.
 */
int oracle_swa_rows_given_q(const oracle_shape* s, int64_t T, const void* qrows,
                            const void* k, const void* v, const void* alpha,
                            const void* beta, int64_t n_rows, const int64_t* rows,
                            double* out)
{
    if (!s || s->head_dim > 512 || s->n_kv_heads < 1 ||
        s->n_q_heads % s->n_kv_heads || s->window < 1)
        return -1;
    for (int64_t u = 0; u < n_rows; ++u)
        if (rows[3 * u] < 0 || rows[3 * u] >= s->batch || rows[3 * u + 1] < 0 ||
            rows[3 * u + 1] >= T || rows[3 * u + 2] < 0 || rows[3 * u + 2] >= s->n_q_heads)
            return -1;
    rows_ctx c = {s, T, qrows, k, v, alpha, beta, rows, out};
    parallel_for(s->nthreads, n_rows, rows_given_q_unit, &c);
    return 0;
}

/* -------------------------------------------------------------- decode */

typedef struct {
    const oracle_shape* s;
    int64_t cap;
    const void *q, *q_out, *alpha, *beta, *alpha_out, *beta_out;
    const void *k_cache, *v_cache;
    const int32_t* len; /* lengths before the step */
    double *o, *o_out;
} decode_ctx;

/* Unit = (b, h): base token at position L = len[b] reads its window
 * [max(0, L-w+1), L]; its output copy reads [0, L] ([N] §2.5, decode row). */
static void decode_unit(void* p, int64_t u)
{
    decode_ctx* c = (decode_ctx*)p;
    const oracle_shape* s = c->s;
    int Hq = s->n_q_heads, Hkv = s->n_kv_heads, d = s->head_dim;
    int64_t b = u / Hq;
    int h = (int)(u % Hq), g = h / (Hq / Hkv);
    int64_t L = c->len[b];
    int64_t base = (b * Hkv + g) * c->cap * d;
    double qh[512];
    if (c->o) {
        scale_offset(c->q, (b * Hq + h) * d, c->alpha, c->beta, h, d, s->dtype, qh);
        int64_t lo = L - s->window + 1;
        if (lo < 0) lo = 0;
        attend(qh, d, s->softmax_scale, c->k_cache, c->v_cache, s->dtype, base, d,
               lo, L, c->o + (b * Hq + h) * d);
    }
    if (c->o_out) {
        scale_offset(c->q_out, (b * Hq + h) * d, c->alpha_out, c->beta_out, h, d,
                     s->dtype, qh);
        attend(qh, d, s->softmax_scale, c->k_cache, c->v_cache, s->dtype, base, d,
               0, L, c->o_out + (b * Hq + h) * d);
    }
}

/*
 * One decode step.  For each sequence b with L = cache_len[b]: the new
 * base token's K/V (k_new, v_new [B][Hkv][d]) are written to slot L; the
 * base query (q [B][Hq][d]) attends over its window, the output copy
 * (q_out [B][Hq][d]) over the whole history [0, L]; then cache_len[b] =
 * L + 1.  With o and o_out both NULL only the append and the length update
 * happen.  Returns -1 when a slot L >= cap or head_dim > 512.
 */
int oracle_decode_step(const oracle_shape* s, const void* q, const void* q_out,
                       const void* k_new, const void* v_new,
                       const void* alpha, const void* beta,
                       const void* alpha_out, const void* beta_out,
                       void* k_cache, void* v_cache, int64_t cap,
                       int32_t* cache_len, double* o, double* o_out)
{
    if (!s || s->head_dim > 512 || s->n_kv_heads < 1 ||
        s->n_q_heads % s->n_kv_heads || s->window < 1)
        return -1;
    int Hq = s->n_q_heads, Hkv = s->n_kv_heads, d = s->head_dim;
    size_t es = elem_size(s->dtype), row = (size_t)d * es;
    for (int b = 0; b < s->batch; ++b)
        if (cache_len[b] < 0 || cache_len[b] >= cap) return -1;

    /* Append first: the copy's key set j <= L includes the new token
     * ([N] §2.4 walk-through: C' reads K_C). */
    for (int64_t b = 0; b < s->batch; ++b)
        for (int g = 0; g < Hkv; ++g) {
            size_t src = (size_t)((b * Hkv + g) * d) * es;
            size_t dst = (size_t)(((b * Hkv + g) * cap + cache_len[b]) * d) * es;
            memcpy((char*)k_cache + dst, (const char*)k_new + src, row);
            memcpy((char*)v_cache + dst, (const char*)v_new + src, row);
        }
    if (o || o_out) {
        decode_ctx c = {s, cap, q, q_out, alpha, beta, alpha_out, beta_out,
                        k_cache, v_cache, cache_len, o, o_out};
        parallel_for(s->nthreads, (int64_t)s->batch * Hq, decode_unit, &c);
    }
    for (int b = 0; b < s->batch; ++b) cache_len[b] += 1;
    return 0;
}

int oracle_version(void) { return 1; }
