/*
 * dsa_oracle.c -- plain fp64 reference for the DSA path (see dsa_oracle.h
 * for the sources [R], [M], [S]).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the library.  Every function is the
 * plain definition written out with nested loops in fp64; nothing is blocked,
 * fused or reordered.  Query rows are spread over threads, each row is
 * computed start-to-finish by one thread in a fixed order, so the result does
 * not depend on the thread count.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -shared -fPIC -pthread -lm
 */
#include "dsa_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Element decoders, written from the bit layouts.                           */
/* ------------------------------------------------------------------------ */

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 mantissa bits. */
static double bf16_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int m = h & 0x7f;
    double v;
    if (e == 0xff)
        v = (m == 0) ? INFINITY : NAN;
    else if (e == 0)
        v = ldexp((double)m, -126 - 7);              /* subnormal: m/128 * 2^-126 */
    else
        v = ldexp(1.0 + (double)m / 128.0, e - 127);
    return sign ? -v : v;
}

/* OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no
 * infinities, S.1111.111 is NaN, largest finite value 448. */
static double e4m3_value(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xf;
    int m = c & 0x7;
    double v;
    if (e == 0xf && m == 0x7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -6 - 3);                /* subnormal: m/8 * 2^-6 */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

void oref_bf16_to_f64(const uint16_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = bf16_value(src[i]);
}

void oref_e4m3_to_f64(const uint8_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = e4m3_value(src[i]);
}

/* Element i of an array of the given encoding, as fp64. */
static double elem(int dtype, const void *base, int64_t i)
{
    switch (dtype) {
    case OREF_F32: return (double)((const float *)base)[i];
    case OREF_BF16: return bf16_value(((const uint16_t *)base)[i]);
    default: return e4m3_value(((const uint8_t *)base)[i]);
    }
}

/* ------------------------------------------------------------------------ */
/* Cache addressing.  Paged layout: fixed-size token pages reached through a  */
/* per-sequence page table ([S] section 5.3: page size 64).                  */
/* ------------------------------------------------------------------------ */

int64_t oref_cache_row(const oref_rows *rows, int32_t b, int64_t s)
{
    if (rows->page_table) {
        int64_t page = rows->page_table[(int64_t)b * rows->max_pages + s / rows->page_size];
        return page * rows->page_size + s % rows->page_size;
    }
    return rows->seq_start[b] + s;
}

/* ------------------------------------------------------------------------ */
/* A tiny fork/join helper: thread t handles list items i with i % T == t.   */
/* ------------------------------------------------------------------------ */

typedef void (*row_fn)(void *ctx, int32_t i);
typedef struct { row_fn fn; void *ctx; int32_t n, t, T; } worker_arg;

static void *worker(void *p)
{
    worker_arg *a = (worker_arg *)p;
    for (int32_t i = a->t; i < a->n; i += a->T) a->fn(a->ctx, i);
    return NULL;
}

static void run_rows(row_fn fn, void *ctx, int32_t n, int n_threads)
{
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    if (n_threads > n) n_threads = n > 0 ? n : 1;
    if (n_threads == 1) {
        for (int32_t i = 0; i < n; ++i) fn(ctx, i);
        return;
    }
    pthread_t th[256];
    worker_arg args[256];
    for (int t = 0; t < n_threads; ++t) {
        args[t] = (worker_arg){fn, ctx, n, t, n_threads};
        pthread_create(&th[t], NULL, worker, &args[t]);
    }
    for (int t = 0; t < n_threads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* Lightning indexer ([R] ①):                                                */
/*   I[t,s] = sum_j w[t,j] * ReLU(q[t,j,:] . k[s,:])                         */
/* over the preceding tokens s of the query's sequence (self included).      */
/* One key per token, shared by all indexer heads (k carries no head index). */
/* FP8 inputs are dequantised literally: value = decode(code) * scale, with  */
/* a scale per (row, head) for q and per cache row for k.                    */
/* ------------------------------------------------------------------------ */

typedef struct {
    int dtype, H, D;
    const void *q; const float *q_scale; const float *w;
    const void *k; const float *k_scale;
    const oref_rows *rows; const int32_t *which;
    double *out; int64_t ld;
} idx_ctx;

static void indexer_row(void *p, int32_t i)
{
    const idx_ctx *c = (const idx_ctx *)p;
    const int32_t r = c->which[i];
    const int32_t b = c->rows->row_seq[r];
    const int64_t n = c->rows->row_len[r];
    const int H = c->H, D = c->D;
    double *qv = (double *)malloc(sizeof(double) * (size_t)H * D);
    double *kv = (double *)malloc(sizeof(double) * (size_t)D);
    for (int j = 0; j < H; ++j) {
        double sq = (c->dtype == OREF_E4M3) ? (double)c->q_scale[(int64_t)r * H + j] : 1.0;
        for (int d = 0; d < D; ++d)
            qv[j * D + d] = elem(c->dtype, c->q, ((int64_t)r * H + j) * D + d) * sq;
    }
    for (int64_t s = 0; s < n; ++s) {
        int64_t row = oref_cache_row(c->rows, b, s);
        double sk = (c->dtype == OREF_E4M3) ? (double)c->k_scale[row] : 1.0;
        for (int d = 0; d < D; ++d) kv[d] = elem(c->dtype, c->k, row * D + d) * sk;
        double x = 0.0;
        for (int j = 0; j < H; ++j) {
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += qv[j * D + d] * kv[d];
            double relu = dot > 0.0 ? dot : 0.0;
            x += (double)c->w[(int64_t)r * H + j] * relu;
        }
        c->out[(int64_t)i * c->ld + s] = x;
    }
    free(qv);
    free(kv);
}

int oref_indexer(int dtype, int n_heads, int head_dim,
                 const void *q, const float *q_scale, const float *w,
                 const void *k, const float *k_scale,
                 const oref_rows *rows, const int32_t *which, int32_t n_which,
                 double *out, int64_t ld, int n_threads)
{
    if (dtype < OREF_F32 || dtype > OREF_E4M3 || n_heads <= 0 || head_dim <= 0) return 1;
    if (dtype == OREF_E4M3 && (!q_scale || !k_scale)) return 1;
    idx_ctx c = {dtype, n_heads, head_dim, q, q_scale, w, k, k_scale, rows, which, out, ld};
    run_rows(indexer_row, &c, n_which, n_threads);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Fine-grained token selection ([R] ②; [M] "Indexer-selected sparse         */
/* attention": k is capped at the row length, indices are int32).           */
/* Order positions by score descending, then position ascending (the lower   */
/* position wins a tie; -0 and +0 compare equal as doubles), keep the first  */
/* k_eff = min(k, n).  The result is a set; it is written in ascending       */
/* position order and padded with -1.                                        */
/* ------------------------------------------------------------------------ */

typedef struct { double v; int32_t pos; } scored;

static int by_score_then_pos(const void *a, const void *b)
{
    const scored *x = (const scored *)a, *y = (const scored *)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->pos > y->pos) - (x->pos < y->pos);
}

static int ascending_i32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

int oref_topk_row(const double *x, int64_t n, int32_t k, int32_t *out)
{
    int64_t keff = n < k ? n : k;
    scored *all = (scored *)malloc(sizeof(scored) * (size_t)(n > 0 ? n : 1));
    for (int64_t s = 0; s < n; ++s) { all[s].v = x[s]; all[s].pos = (int32_t)s; }
    qsort(all, (size_t)n, sizeof(scored), by_score_then_pos);
    for (int64_t i = 0; i < keff; ++i) out[i] = all[i].pos;
    qsort(out, (size_t)keff, sizeof(int32_t), ascending_i32);
    for (int64_t i = keff; i < k; ++i) out[i] = -1;
    free(all);
    return (int)keff;
}

typedef struct {
    const double *x; const float *xf; int64_t ld; const int32_t *len; int32_t k; int32_t *out;
} topk_ctx;

static void topk_row_job(void *p, int32_t r)
{
    const topk_ctx *c = (const topk_ctx *)p;
    int64_t n = c->len[r];
    if (c->x) {
        oref_topk_row(c->x + (int64_t)r * c->ld, n, c->k, c->out + (int64_t)r * c->k);
    } else {
        double *row = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        for (int64_t s = 0; s < n; ++s) row[s] = (double)c->xf[(int64_t)r * c->ld + s];
        oref_topk_row(row, n, c->k, c->out + (int64_t)r * c->k);
        free(row);
    }
}

int oref_topk_rows(const double *x, int64_t ld, const int32_t *len, int32_t n_rows,
                   int32_t k, int32_t *out, int n_threads)
{
    if (k <= 0) return 1;
    topk_ctx c = {x, NULL, ld, len, k, out};
    run_rows(topk_row_job, &c, n_rows, n_threads);
    return 0;
}

int oref_topk_rows_f32(const float *x, int64_t ld, const int32_t *len, int32_t n_rows,
                       int32_t k, int32_t *out, int n_threads)
{
    if (k <= 0) return 1;
    topk_ctx c = {NULL, x, ld, len, k, out};
    run_rows(topk_row_job, &c, n_rows, n_threads);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention in MQA mode ([R], MLA-based implementation: every latent entry  */
/* is shared by all query heads; [M] "Multi-head latent attention": the      */
/* entry is the kv_lora_rank latent followed by the RoPE key).  Keys are the */
/* full d_qk-wide entries, values are the first d_v dims (the latent).  Plain */
/* softmax with no sink term and no output gate ([M] "Learnable attention    */
/* sink", "Gated attention output": both absent).                            */
/*   z_s = scale * q_h . C_s ;  o_h = sum_s softmax(z)_s * C_s[0:d_v] ;      */
/*   lse_h = ln sum_s exp(z_s)                                              */
/* ------------------------------------------------------------------------ */

typedef struct {
    int dtype, H, Dqk, Dv; double scale;
    const void *q; const void *kv; const int32_t *idx; int32_t k;
    const oref_rows *rows; const int32_t *which;
    double *out; double *lse;
} mla_ctx;

static void attend_row(const mla_ctx *c, int32_t i, const int64_t *pos, int64_t n_pos)
{
    const int32_t r = c->which[i];
    const int32_t b = c->rows->row_seq[r];
    const int H = c->H, Dqk = c->Dqk, Dv = c->Dv;
    double *ent = (double *)malloc(sizeof(double) * (size_t)(n_pos > 0 ? n_pos : 1) * Dqk);
    double *z = (double *)malloc(sizeof(double) * (size_t)(n_pos > 0 ? n_pos : 1));
    double *qh = (double *)malloc(sizeof(double) * (size_t)Dqk);
    for (int64_t e = 0; e < n_pos; ++e) {
        int64_t row = oref_cache_row(c->rows, b, pos[e]);
        for (int d = 0; d < Dqk; ++d) ent[e * Dqk + d] = elem(c->dtype, c->kv, row * Dqk + d);
    }
    for (int h = 0; h < H; ++h) {
        double *o = c->out + ((int64_t)i * H + h) * Dv;
        for (int d = 0; d < Dqk; ++d) qh[d] = elem(c->dtype, c->q, ((int64_t)r * H + h) * Dqk + d);
        if (n_pos == 0) {
            for (int d = 0; d < Dv; ++d) o[d] = 0.0;
            if (c->lse) c->lse[(int64_t)i * H + h] = -INFINITY;
            continue;
        }
        double m = -INFINITY;
        for (int64_t e = 0; e < n_pos; ++e) {
            double dot = 0.0;
            for (int d = 0; d < Dqk; ++d) dot += qh[d] * ent[e * Dqk + d];
            z[e] = c->scale * dot;
            if (z[e] > m) m = z[e];
        }
        double l = 0.0;
        for (int64_t e = 0; e < n_pos; ++e) {
            z[e] = exp(z[e] - m);                    /* unnormalised weight e^{z-m} */
            l += z[e];
        }
        for (int d = 0; d < Dv; ++d) {
            double acc = 0.0;
            for (int64_t e = 0; e < n_pos; ++e) acc += z[e] * ent[e * Dqk + d];
            o[d] = acc / l;
        }
        if (c->lse) c->lse[(int64_t)i * H + h] = m + log(l);
    }
    free(ent);
    free(z);
    free(qh);
}

/* idx entries that are negative or not below the row length are skipped;
 * duplicates (never produced by top-k) would be counted once per occurrence. */
static void sparse_row(void *p, int32_t i)
{
    const mla_ctx *c = (const mla_ctx *)p;
    const int32_t r = c->which[i];
    const int64_t n = c->rows->row_len[r];
    int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * (size_t)c->k);
    int64_t n_pos = 0;
    for (int32_t j = 0; j < c->k; ++j) {
        int64_t s = c->idx[(int64_t)r * c->k + j];
        if (s >= 0 && s < n) pos[n_pos++] = s;
    }
    attend_row(c, i, pos, n_pos);
    free(pos);
}

static void dense_row(void *p, int32_t i)
{
    const mla_ctx *c = (const mla_ctx *)p;
    const int64_t n = c->rows->row_len[c->which[i]];
    int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t s = 0; s < n; ++s) pos[s] = s;
    attend_row(c, i, pos, n);
    free(pos);
}

int oref_sparse_mla(int dtype, int n_heads, int d_qk, int d_v, double scale,
                    const void *q, const void *kv, const int32_t *idx, int32_t k,
                    const oref_rows *rows, const int32_t *which, int32_t n_which,
                    double *out, double *lse, int n_threads)
{
    if (dtype < OREF_F32 || dtype > OREF_BF16 || n_heads <= 0 || d_qk <= 0 || d_v <= 0 ||
        d_v > d_qk || k <= 0)
        return 1;
    mla_ctx c = {dtype, n_heads, d_qk, d_v, scale, q, kv, idx, k, rows, which, out, lse};
    run_rows(sparse_row, &c, n_which, n_threads);
    return 0;
}

int oref_dense_mqa(int dtype, int n_heads, int d_qk, int d_v, double scale,
                   const void *q, const void *kv,
                   const oref_rows *rows, const int32_t *which, int32_t n_which,
                   double *out, double *lse, int n_threads)
{
    if (dtype < OREF_F32 || dtype > OREF_BF16 || n_heads <= 0 || d_qk <= 0 || d_v <= 0 ||
        d_v > d_qk)
        return 1;
    mla_ctx c = {dtype, n_heads, d_qk, d_v, scale, q, kv, NULL, 0, rows, which, out, lse};
    run_rows(dense_row, &c, n_which, n_threads);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Indexer-input and cache-write prep (definitions in dsa_oracle.h).         */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t bits_of_f32(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* The two bf16 values around f are f with its low 16 bits cleared (toward
 * zero) and the next one away from zero; take the nearer, ties to the even
 * code. */
uint16_t oref_bf16_code(float f)
{
    if (isnan(f)) return 0x7fc0;
    const uint32_t u = bits_of_f32(f);
    const uint32_t lo = u & 0xffff0000u;
    const uint32_t hi = lo + 0x10000u;
    const double v = fabs((double)f);
    const double vlo = fabs((double)f32_from_bits(lo));
    const double vhi = ((hi >> 23) & 0xff) == 0xff ? INFINITY : fabs((double)f32_from_bits(hi));
    const double dlo = v - vlo, dhi = vhi - v;
    if (dlo < dhi) return (uint16_t)(lo >> 16);
    if (dhi < dlo) return (uint16_t)(hi >> 16);
    return ((lo >> 16) & 1) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);
}

/* Search of the 127 finite non-negative e4m3 codes for the nearest value. */
uint8_t oref_e4m3_code(float f)
{
    const double v = fabs((double)f);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7e; ++c) {
        const double d = fabs(e4m3_value((uint8_t)c) - v);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(signbit(f) ? (best | 0x80) : best);
}

/* One rotated pair, every product and sum rounded to fp32 once. */
static void rope_pair(float a, float b, float c, float s, float *ya, float *yb)
{
    const float ac = a * c, bs = b * s, bc = b * c, as = a * s;
    *ya = ac - bs;
    *yb = bc + as;
}

static float bf16_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* A 128-dim indexer vector: dims 0..63 rotated non-interleaved, the rest kept;
 * written as bf16 codes or as e4m3 codes with their scale. */
static void indexer_vector(const uint16_t *in, const float *cs, int idx_dtype, void *out,
                           float *scale_out)
{
    float y[128];
    for (int j = 0; j < 128; ++j) y[j] = bf16_f32(in[j]);
    for (int i = 0; i < 32; ++i) {
        float a, b;
        rope_pair(y[i], y[i + 32], cs[i], cs[32 + i], &a, &b);
        y[i] = a;
        y[i + 32] = b;
    }
    if (idx_dtype == OREF_BF16) {
        uint16_t *o = (uint16_t *)out;
        for (int j = 0; j < 128; ++j) o[j] = j < 64 ? oref_bf16_code(y[j]) : in[j];
        return;
    }
    float amax = 0.0f;
    for (int j = 0; j < 128; ++j)
        if (fabsf(y[j]) > amax) amax = fabsf(y[j]);
    const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    uint8_t *o = (uint8_t *)out;
    for (int j = 0; j < 128; ++j) o[j] = oref_e4m3_code(y[j] / scale);
    *scale_out = scale;
}

/* A 576-dim MLA vector: dims 512..575 rotated interleaved, the rest kept. */
static void mla_vector(const uint16_t *in, const float *cs, uint16_t *out)
{
    for (int j = 0; j < 512; ++j) out[j] = in[j];
    for (int i = 0; i < 32; ++i) {
        float a, b;
        rope_pair(bf16_f32(in[512 + 2 * i]), bf16_f32(in[513 + 2 * i]), cs[i], cs[32 + i], &a, &b);
        out[512 + 2 * i] = oref_bf16_code(a);
        out[513 + 2 * i] = oref_bf16_code(b);
    }
}

int oref_prep_keys(int32_t n_tok, const int32_t *pos, const int64_t *rows_out, int64_t cache_rows,
                   const float *cos_sin, int32_t max_pos, int idx_dtype,
                   const uint16_t *k_in, void *k_cache, float *k_scale,
                   const uint16_t *kv_in, uint16_t *kv_cache)
{
    if (n_tok < 0 || max_pos <= 0 || (idx_dtype != OREF_BF16 && idx_dtype != OREF_E4M3))
        return 1;
    const size_t elt = idx_dtype == OREF_BF16 ? 2 : 1;
    for (int32_t t = 0; t < n_tok; ++t) {
        const int32_t p = pos[t];
        const int64_t r = rows_out[t];
        if (p < 0 || p >= max_pos || r < 0 || r >= cache_rows) continue;
        const float *cs = cos_sin + (int64_t)p * 64;
        indexer_vector(k_in + (int64_t)t * 128, cs, idx_dtype,
                       (uint8_t *)k_cache + (size_t)r * 128 * elt, k_scale ? k_scale + r : NULL);
        mla_vector(kv_in + (int64_t)t * 576, cs, kv_cache + (size_t)r * 576);
    }
    return 0;
}

int oref_prep_queries(int32_t n_rows, const int32_t *pos, const float *cos_sin, int32_t max_pos,
                      int idx_dtype, int32_t n_idx_heads, const uint16_t *qi_in, void *qi_out,
                      float *qi_scale, int32_t n_heads, uint16_t *q)
{
    if (n_rows < 0 || max_pos <= 0 || n_idx_heads <= 0 || n_heads <= 0 ||
        (idx_dtype != OREF_BF16 && idx_dtype != OREF_E4M3))
        return 1;
    const size_t elt = idx_dtype == OREF_BF16 ? 2 : 1;
    uint16_t *tmp = (uint16_t *)malloc(576 * sizeof(uint16_t));
    if (!tmp) return 2;
    for (int32_t r = 0; r < n_rows; ++r) {
        const int32_t p = pos[r];
        if (p < 0 || p >= max_pos) continue;
        const float *cs = cos_sin + (int64_t)p * 64;
        for (int32_t h = 0; h < n_idx_heads; ++h) {
            const int64_t v = (int64_t)r * n_idx_heads + h;
            indexer_vector(qi_in + v * 128, cs, idx_dtype, (uint8_t *)qi_out + (size_t)v * 128 * elt,
                           qi_scale ? qi_scale + v : NULL);
        }
        for (int32_t h = 0; h < n_heads; ++h) {
            uint16_t *qh = q + ((int64_t)r * n_heads + h) * 576;
            mla_vector(qh, cs, tmp);
            memcpy(qh, tmp, 576 * sizeof(uint16_t));
        }
    }
    free(tmp);
    return 0;
}

void oref_bf16_codes(const float *src, uint16_t *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = oref_bf16_code(src[i]);
}

void oref_e4m3_codes(const float *src, uint8_t *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = oref_e4m3_code(src[i]);
}

/* ------------------------------------------------------------------------ */
/* Masked MHA mode for short prefill ([R], "短序列优化": short prefill runs  */
/* DSA as masked MHA).  Per head h the latent entry c_s (512) and RoPE key   */
/* kr_s (64) of position s give the 192-dim key [W_UK[h] c_s | kr_s] and the */
/* 128-dim value W_UV[h] c_s ([M] "Multi-head latent attention": 128 heads,  */
/* 128 nope + 64 rope query/key dims, 128 value dims).  A row attends over   */
/* its top-k positions (as a set), or over every position below its length  */
/* when no idx is given (dense causal: what the top-k selects whenever the  */
/* row has at most k positions).                                             */
/* ------------------------------------------------------------------------ */

typedef struct {
    int H;
    const uint16_t *kv, *w_uk, *w_uv;
    double *k, *v;
} decomp_ctx;

static void decompress_row(void *p, int32_t n)
{
    const decomp_ctx *c = (const decomp_ctx *)p;
    double lat[576];
    for (int j = 0; j < 576; ++j) lat[j] = bf16_value(c->kv[(int64_t)n * 576 + j]);
    for (int h = 0; h < c->H; ++h) {
        double *kk = c->k + ((int64_t)n * c->H + h) * 192;
        double *vv = c->v + ((int64_t)n * c->H + h) * 128;
        for (int d = 0; d < 128; ++d) {
            const uint16_t *wk = c->w_uk + ((int64_t)h * 128 + d) * 512;
            const uint16_t *wv = c->w_uv + ((int64_t)h * 128 + d) * 512;
            double sk = 0.0, sv = 0.0;
            for (int j = 0; j < 512; ++j) {
                sk += bf16_value(wk[j]) * lat[j];
                sv += bf16_value(wv[j]) * lat[j];
            }
            kk[d] = sk;
            vv[d] = sv;
        }
        for (int d = 0; d < 64; ++d) kk[128 + d] = lat[512 + d];
    }
}

int oref_mha_decompress(int32_t n_cache_rows, int n_heads, const uint16_t *kv, const uint16_t *w_uk,
                        const uint16_t *w_uv, double *k, double *v, int n_threads)
{
    if (n_cache_rows < 0 || n_heads <= 0) return 1;
    decomp_ctx c = {n_heads, kv, w_uk, w_uv, k, v};
    run_rows(decompress_row, &c, n_cache_rows, n_threads);
    return 0;
}

typedef struct {
    int H;
    const uint16_t *q;
    const double *k, *v;
    const oref_rows *rows;
    const int32_t *idx;
    int32_t topk;
    double scale;
    const int32_t *which;
    double *out, *lse;
} mha_ctx;

static void mha_row(void *p, int32_t i)
{
    const mha_ctx *c = (const mha_ctx *)p;
    const int32_t r = c->which[i];
    const int32_t b = c->rows->row_seq[r];
    const int64_t n = c->rows->row_len[r];
    /* the attended positions: the set of valid idx entries, or 0 .. n-1 */
    unsigned char *in = (unsigned char *)calloc((size_t)(n > 0 ? n : 1), 1);
    for (int64_t s = 0; s < n; ++s) in[s] = c->idx ? 0 : 1;
    if (c->idx)
        for (int32_t j = 0; j < c->topk; ++j) {
            const int64_t s = c->idx[(int64_t)r * c->topk + j];
            if (s >= 0 && s < n) in[s] = 1;
        }
    double *z = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int h = 0; h < c->H; ++h) {
        double qh[192];
        for (int d = 0; d < 192; ++d) qh[d] = bf16_value(c->q[((int64_t)r * c->H + h) * 192 + d]);
        double *o = c->out + ((int64_t)i * c->H + h) * 128;
        double m = -INFINITY;
        for (int64_t s = 0; s < n; ++s) {
            if (!in[s]) continue;
            const double *kk = c->k + (oref_cache_row(c->rows, b, s) * c->H + h) * 192;
            double dot = 0.0;
            for (int d = 0; d < 192; ++d) dot += qh[d] * kk[d];
            z[s] = c->scale * dot;
            if (z[s] > m) m = z[s];
        }
        double l = 0.0;
        for (int d = 0; d < 128; ++d) o[d] = 0.0;
        for (int64_t s = 0; s < n; ++s) {
            if (!in[s]) continue;
            const double w = exp(z[s] - m);
            const double *vv = c->v + (oref_cache_row(c->rows, b, s) * c->H + h) * 128;
            l += w;
            for (int d = 0; d < 128; ++d) o[d] += w * vv[d];
        }
        if (l > 0.0)
            for (int d = 0; d < 128; ++d) o[d] /= l;
        if (c->lse) c->lse[(int64_t)i * c->H + h] = l > 0.0 ? m + log(l) : -INFINITY;
    }
    free(z);
    free(in);
}

int oref_mha(int n_heads, const uint16_t *q, const double *k, const double *v,
             const oref_rows *rows, const int32_t *idx, int32_t topk, double scale,
             const int32_t *which, int32_t n_which, double *out, double *lse, int n_threads)
{
    if (n_heads <= 0 || (idx && topk <= 0)) return 1;
    mha_ctx c = {n_heads, q, k, v, rows, idx, topk, scale, which, out, lse};
    run_rows(mha_row, &c, n_which, n_threads);
    return 0;
}
