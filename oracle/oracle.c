/*
 * oracle.c -- plain fp64 CPU reference for exact softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU path never calls it
 * and shares no code with it.
 *
 * What it computes is the plain definition, which FlashAttention reaches
 * without approximation: the tiled kernel and standard attention agree up to
 * rounding ("FlashAttention Explained", section "Online softmax"; "Flash
 * Attention and Memory-Efficient Attention Variants", worked example).  Per
 * head, with S = scale * Q K^T:
 *
 *   P   = softmax(S) row-wise, over visible keys only
 *   O   = P V
 *   L_i = m_i + ln(sum_j exp(S_ij - m_i))        (natural-log logsumexp)
 *
 * The backward is the analytic derivative of O with respect to Q, K, V as
 * outlined on the "FlashAttention" deep-dive page (section "How it works":
 * D = rowsum(dO * O), dS = P * (dP - D)):
 *
 *   dV = P^T dO,   dP = dO V^T,   D_i = sum_t dO_it O_it,
 *   dS = P * (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q.
 *
 * A second forward, oracle_attn_fwd_tiled, reduces each block of keys to a
 * per-row summary (block maximum, sum of exponentials, weighted sum of V) and
 * folds the summaries together with the rescaling rule of the same deep-dive
 * page ("How it works": running maximum and sum, rescale by exp(m_old - m_new),
 * one division at the end), in fp64, so that tiled and untiled results can be
 * compared.  It also records the running state of one chosen row after every
 * key block, which the worked example on the "Flash Attention and
 * Memory-Efficient Attention Variants" page prints.
 *
 * Layout: every tensor is row-major contiguous [BH, N, d] (lse/delta [BH, N]),
 * fp64.  Causal means key j is visible to query i iff j <= i (square,
 * top-left aligned).  A row with no visible key (unreachable for square
 * causal masks) gets O = 0 and L = -inf, as the deep-dive page's pitfalls
 * section prescribes for fully masked rows.
 *
 * Grouped heads (GQA/MQA, "FlashAttention" deep-dive page, "Implementation
 * notes"): the _gqa entry points take Hq query heads and Hkv = Hq / G key/value
 * heads per batch; query head h of batch b attends with key/value head
 * h / G of batch b.  The forward is the plain definition above with that
 * head's K and V; K and V are shared by G query heads, so their gradients are
 * the sums over those heads of the per-head dK and dV.
 *
 * Decode (same page, "Implementation notes"): one query row per (batch,
 * query head) against the first kv_len[b] keys of a key/value cache; the
 * plain definition again, see oracle_attn_decode.
 *
 * Parallelism: rows (forward, dQ) or keys (dK, dV) are split over POSIX
 * threads; every output element is computed by exactly one thread in a fixed
 * order, so results do not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

static int resolve_threads(int nthreads) {
    if (nthreads > 0) return nthreads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/* ------------------------------------------------------------------------ */
/* A tiny "parallel for" over [0, count).                                   */

typedef void (*range_fn)(void* ctx, int64_t begin, int64_t end);

typedef struct {
    range_fn fn;
    void* ctx;
    int64_t begin, end;
    int running; /* 1 if a thread was started for this range */
} range_job;

static void* range_thread(void* p) {
    range_job* j = (range_job*)p;
    j->fn(j->ctx, j->begin, j->end);
    return NULL;
}

static int parallel_for(int64_t count, int nthreads, range_fn fn, void* ctx) {
    int nt = resolve_threads(nthreads);
    if ((int64_t)nt > count) nt = (int)(count > 0 ? count : 1);
    if (nt <= 1) {
        fn(ctx, 0, count);
        return ORACLE_OK;
    }
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    range_job* jobs = (range_job*)malloc(sizeof(range_job) * (size_t)nt);
    if (!th || !jobs) {
        free(th);
        free(jobs);
        return ORACLE_ERR_NOMEM;
    }
    for (int t = 0; t < nt; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].begin = count * t / nt;
        jobs[t].end = count * (t + 1) / nt;
        jobs[t].running = pthread_create(&th[t], NULL, range_thread, &jobs[t]) == 0;
        if (!jobs[t].running) fn(ctx, jobs[t].begin, jobs[t].end); /* no thread: do it here */
    }
    for (int t = 0; t < nt; ++t)
        if (jobs[t].running) pthread_join(th[t], NULL);
    free(th);
    free(jobs);
    return ORACLE_OK;
}

static int visible(int causal, int64_t i, int64_t j) { return !causal || j <= i; }

/* ------------------------------------------------------------------------ */
/* Dropout ("FlashAttention" deep-dive page, "Implementation notes": the     */
/* backward regenerates the mask from a Philox seed and offset).             */
/*                                                                           */
/* Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw ("Parallel   */
/* Random Numbers: As Easy as 1, 2, 3", SC 2011): ten rounds of              */
/*   (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, */
/*                        lo(M0 c0))                                         */
/* with M0 = 0xD2511F53, M1 = 0xCD9E8D57, the key (k0, k1) advanced by the    */
/* Weyl constants (0x9E3779B9, 0xBB67AE85) before every round but the first. */
/*                                                                           */
/* Element (bh, i, j) -- flat query head bh, query row i, key j -- reads the */
/* byte 8 (j mod 4) of word (j / 8) mod 4 of                                 */
/*   Philox(counter = (2 (j / 32) + (j / 4) mod 2, i, bh, offset),           */
/*          key = (seed mod 2^32, seed / 2^32))                              */
/* and is kept when that byte is >= thr = floor(256 p + 1/2); kept           */
/* probabilities are scaled by 256 / (256 - thr), so the drop probability is */
/* thr / 256.  L and the softmax denominator are those of the undropped P.    */
/* The pages print no Philox output; the generator is pinned to the known-   */
/* answer vectors published with the Random123 reference implementation of  */
/* the same paper (oracle_philox4x32_10 exports it for that check).          */

typedef struct {
    int thr;           /* bytes below thr are dropped */
    double keep_scale; /* 256 / (256 - thr) */
    uint32_t k0, k1;   /* Philox key: the seed */
    uint32_t offset;   /* fourth counter word */
} dropout_cfg;

static void philox4x32_10(const uint32_t ctr[4], uint32_t k0, uint32_t k1, uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* The generator itself, for its known-answer check: out = Philox4x32-10(ctr, key). */
int oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    if (!ctr || !key || !out) return ORACLE_ERR_ARG;
    philox4x32_10(ctr, key[0], key[1], out);
    return ORACLE_OK;
}

static unsigned dropout_byte(const dropout_cfg* dc, int64_t bh, int64_t i, int64_t j) {
    const uint32_t ctr[4] = {(uint32_t)(2 * (j / 32) + ((j / 4) & 1)), (uint32_t)i, (uint32_t)bh, dc->offset};
    uint32_t w[4];
    philox4x32_10(ctr, dc->k0, dc->k1, w);
    return (w[(j / 8) & 3] >> (8 * (j & 3))) & 0xFFu;
}

/* The factor element (bh, i, j) of P is multiplied by: 0 (dropped) or the keep scale. */
static double dropout_factor(const dropout_cfg* dc, int64_t bh, int64_t i, int64_t j) {
    if (!dc) return 1.0;
    return dropout_byte(dc, bh, i, j) >= (unsigned)dc->thr ? dc->keep_scale : 0.0;
}

static int dropout_setup(dropout_cfg* dc, double p, uint64_t seed, uint64_t offset) {
    if (!(p >= 0.0 && p < 1.0) || offset > 0xFFFFFFFFull) return ORACLE_ERR_ARG;
    int thr = (int)floor(256.0 * p + 0.5);
    if (thr > 255) thr = 255;
    dc->thr = thr;
    dc->keep_scale = 256.0 / (256.0 - thr);
    dc->k0 = (uint32_t)seed;
    dc->k1 = (uint32_t)(seed >> 32);
    dc->offset = (uint32_t)offset;
    return ORACLE_OK;
}

/* Keep mask (1 kept, 0 dropped) of query heads bh < BH, rows i < N, keys j < N. */
int oracle_dropout_mask(uint8_t* mask, int64_t BH, int64_t N, double p, uint64_t seed, uint64_t offset) {
    dropout_cfg dc;
    if (!mask || BH <= 0 || N <= 0 || dropout_setup(&dc, p, seed, offset) != ORACLE_OK) return ORACLE_ERR_ARG;
    for (int64_t bh = 0; bh < BH; ++bh)
        for (int64_t i = 0; i < N; ++i)
            for (int64_t j = 0; j < N; ++j) mask[(bh * N + i) * N + j] = dropout_factor(&dc, bh, i, j) != 0.0;
    return ORACLE_OK;
}

/* The dropout byte itself, for statistical checks of the generator. */
int oracle_dropout_bytes(uint8_t* out, int64_t BH, int64_t N, uint64_t seed, uint64_t offset) {
    dropout_cfg dc;
    if (!out || BH <= 0 || N <= 0 || dropout_setup(&dc, 0.0, seed, offset) != ORACLE_OK) return ORACLE_ERR_ARG;
    for (int64_t bh = 0; bh < BH; ++bh)
        for (int64_t i = 0; i < N; ++i)
            for (int64_t j = 0; j < N; ++j) out[(bh * N + i) * N + j] = (uint8_t)dropout_byte(&dc, bh, i, j);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Forward: the plain definition, one query row at a time.                   */

typedef struct {
    const double *q, *k, *v;
    double *o, *lse;
    int64_t N, d;
    double scale;
    int causal;
    int64_t hq, group; /* query heads per batch, query heads per key/value head */
    const dropout_cfg* drop; /* NULL: no dropout */
} fwd_ctx;

/* Key/value head (flat over batches) read by flat query head bh. */
static int64_t kv_head(int64_t bh, int64_t hq, int64_t group) {
    return (bh / hq) * (hq / group) + (bh % hq) / group;
}

/* One query row r = bh * N + i: scores of the visible keys, their maximum,
 * the softmax denominator, O_i = sum_j softmax_ij v_j and L_i = m + ln l. */
static void fwd_one_row(const fwd_ctx* c, int64_t r, double* s, double* oi, double* lse_out) {
    const int64_t N = c->N, d = c->d;
    const int64_t bh = r / N, i = r % N;
    const int64_t kvh = kv_head(bh, c->hq, c->group);
    const double* qi = c->q + r * d;
    const double* kh = c->k + kvh * N * d;
    const double* vh = c->v + kvh * N * d;
    double m = -INFINITY;
    for (int64_t j = 0; j < N; ++j) {
        if (!visible(c->causal, i, j)) continue;
        double dot = 0.0;
        for (int64_t t = 0; t < d; ++t) dot += qi[t] * kh[j * d + t];
        s[j] = c->scale * dot;
        if (s[j] > m) m = s[j];
    }
    for (int64_t t = 0; t < d; ++t) oi[t] = 0.0;
    if (m == -INFINITY) { /* no visible key: O = 0, L = -inf */
        *lse_out = -INFINITY;
        return;
    }
    double l = 0.0;
    for (int64_t j = 0; j < N; ++j)
        if (visible(c->causal, i, j)) l += exp(s[j] - m);
    for (int64_t j = 0; j < N; ++j) {
        if (!visible(c->causal, i, j)) continue;
        const double pij = exp(s[j] - m) / l * dropout_factor(c->drop, bh, i, j);
        for (int64_t t = 0; t < d; ++t) oi[t] += pij * vh[j * d + t];
    }
    *lse_out = m + log(l);
}

static void fwd_rows(void* p, int64_t begin, int64_t end) {
    fwd_ctx* c = (fwd_ctx*)p;
    double* s = (double*)malloc(sizeof(double) * (size_t)c->N);
    for (int64_t r = begin; r < end; ++r) fwd_one_row(c, r, s, c->o + r * c->d, c->lse + r);
    free(s);
}

typedef struct {
    fwd_ctx base;
    const int64_t* rows;
} fwd_rows_ctx;

static void fwd_listed_rows(void* p, int64_t begin, int64_t end) {
    fwd_rows_ctx* c = (fwd_rows_ctx*)p;
    double* s = (double*)malloc(sizeof(double) * (size_t)c->base.N);
    for (int64_t r = begin; r < end; ++r)
        fwd_one_row(&c->base, c->rows[r], s, c->base.o + r * c->base.d, c->base.lse + r);
    free(s);
}

/* Forward for listed query rows only (rows are independent): rows[r] is a flat
 * index bh * N + i; o receives nrows x d values and lse nrows values. */
int oracle_attn_fwd_rows(const double* q, const double* k, const double* v, const int64_t* rows,
                         int64_t nrows, double* o, double* lse, int64_t BH, int64_t N, int64_t d,
                         double scale, int causal, int nthreads) {
    if (!q || !k || !v || !rows || !o || !lse || BH <= 0 || N <= 0 || d <= 0 || nrows < 0)
        return ORACLE_ERR_ARG;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= BH * N) return ORACLE_ERR_ARG;
    fwd_rows_ctx c = {{q, k, v, o, lse, N, d, scale, causal, BH, 1, NULL}, rows};
    return parallel_for(nrows, nthreads, fwd_listed_rows, &c);
}

/* oracle_attn_fwd_rows with dropout of probability p. */
int oracle_attn_fwd_rows_dropout(const double* q, const double* k, const double* v, const int64_t* rows,
                                 int64_t nrows, double* o, double* lse, int64_t BH, int64_t N, int64_t d,
                                 double scale, int causal, double p, uint64_t seed, uint64_t offset, int nthreads) {
    dropout_cfg dc;
    if (!q || !k || !v || !rows || !o || !lse || BH <= 0 || N <= 0 || d <= 0 || nrows < 0 ||
        dropout_setup(&dc, p, seed, offset) != ORACLE_OK)
        return ORACLE_ERR_ARG;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= BH * N) return ORACLE_ERR_ARG;
    fwd_rows_ctx c = {{q, k, v, o, lse, N, d, scale, causal, BH, 1, &dc}, rows};
    return parallel_for(nrows, nthreads, fwd_listed_rows, &c);
}

int oracle_attn_fwd(const double* q, const double* k, const double* v, double* o, double* lse,
                    int64_t BH, int64_t N, int64_t d, double scale, int causal, int nthreads) {
    if (!q || !k || !v || !o || !lse || BH <= 0 || N <= 0 || d <= 0) return ORACLE_ERR_ARG;
    fwd_ctx c = {q, k, v, o, lse, N, d, scale, causal, BH, 1, NULL};
    return parallel_for(BH * N, nthreads, fwd_rows, &c);
}

/* Grouped-head forward: q, o [B, Hq, N, d], lse [B, Hq, N], k, v [B, Hkv, N, d],
 * Hq a multiple of Hkv. */
int oracle_attn_fwd_gqa(const double* q, const double* k, const double* v, double* o, double* lse,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, double scale,
                        int causal, int nthreads) {
    if (!q || !k || !v || !o || !lse || B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0 ||
        Hq % Hkv != 0)
        return ORACLE_ERR_ARG;
    fwd_ctx c = {q, k, v, o, lse, N, d, scale, causal, Hq, Hq / Hkv, NULL};
    return parallel_for(B * Hq * N, nthreads, fwd_rows, &c);
}

/* Grouped-head forward with dropout of probability p (see dropout_cfg). */
int oracle_attn_fwd_dropout(const double* q, const double* k, const double* v, double* o, double* lse, int64_t B,
                            int64_t Hq, int64_t Hkv, int64_t N, int64_t d, double scale, int causal, double p,
                            uint64_t seed, uint64_t offset, int nthreads) {
    dropout_cfg dc;
    if (!q || !k || !v || !o || !lse || B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0 || Hq % Hkv != 0 ||
        dropout_setup(&dc, p, seed, offset) != ORACLE_OK)
        return ORACLE_ERR_ARG;
    fwd_ctx c = {q, k, v, o, lse, N, d, scale, causal, Hq, Hq / Hkv, &dc};
    return parallel_for(B * Hq * N, nthreads, fwd_rows, &c);
}

/* ------------------------------------------------------------------------ */
/* Decode: one query row per (batch, query head) against a key/value cache   */
/* ("FlashAttention" deep-dive page, "Implementation notes": single-query    */
/* decode over a long cache).  The result is the plain definition: the row   */
/* attends to the first kv_len[b] keys of its key/value head (all Nk when    */
/* kv_len is NULL); no key visible gives O = 0 and L = -inf.                  */

typedef struct {
    const double *q, *k, *v;
    const int64_t* kv_len;
    double *o, *lse;
    int64_t Hq, group, Nk, d;
    double scale;
} dec_ctx;

static void dec_rows(void* p, int64_t begin, int64_t end) {
    const dec_ctx* c = (const dec_ctx*)p;
    const int64_t d = c->d;
    double* s = (double*)malloc(sizeof(double) * (size_t)(c->Nk > 0 ? c->Nk : 1));
    for (int64_t r = begin; r < end; ++r) { /* r = b * Hq + h */
        const int64_t b = r / c->Hq;
        const int64_t n = c->kv_len ? c->kv_len[b] : c->Nk;
        const int64_t kvh = kv_head(r, c->Hq, c->group);
        const double* qr = c->q + r * d;
        const double* kh = c->k + kvh * c->Nk * d;
        const double* vh = c->v + kvh * c->Nk * d;
        double* orow = c->o + r * d;
        double m = -INFINITY;
        for (int64_t j = 0; j < n; ++j) {
            double dot = 0.0;
            for (int64_t t = 0; t < d; ++t) dot += qr[t] * kh[j * d + t];
            s[j] = c->scale * dot;
            if (s[j] > m) m = s[j];
        }
        for (int64_t t = 0; t < d; ++t) orow[t] = 0.0;
        if (n == 0) {
            c->lse[r] = -INFINITY;
            continue;
        }
        double l = 0.0;
        for (int64_t j = 0; j < n; ++j) l += exp(s[j] - m);
        for (int64_t j = 0; j < n; ++j) {
            const double pj = exp(s[j] - m) / l;
            for (int64_t t = 0; t < d; ++t) orow[t] += pj * vh[j * d + t];
        }
        c->lse[r] = m + log(l);
    }
    free(s);
}

/* q, o [B, Hq, d]; lse [B, Hq]; k, v [B, Hkv, Nk, d]; kv_len [B] with
 * 0 <= kv_len[b] <= Nk, or NULL. */
int oracle_attn_decode(const double* q, const double* k, const double* v, const int64_t* kv_len, double* o,
                       double* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nk, int64_t d, double scale,
                       int nthreads) {
    if (!q || !k || !v || !o || !lse || B <= 0 || Hq <= 0 || Hkv <= 0 || Nk <= 0 || d <= 0 || Hq % Hkv != 0)
        return ORACLE_ERR_ARG;
    if (kv_len)
        for (int64_t b = 0; b < B; ++b)
            if (kv_len[b] < 0 || kv_len[b] > Nk) return ORACLE_ERR_ARG;
    dec_ctx c = {q, k, v, kv_len, o, lse, Hq, Hq / Hkv, Nk, d, scale};
    return parallel_for(B * Hq, nthreads, dec_rows, &c);
}

/* ------------------------------------------------------------------------ */
/* Backward: analytic gradients with the full N x N matrices of each head.   */

typedef struct {
    const double *q, *k, *v, *dout;
    double *dq, *dk, *dv, *delta;
    double *P, *dS; /* N x N scratch of the current head */
    double *o, *lse; /* this head's forward outputs */
    int64_t N, d;
    double scale;
    int causal;
    int failed; /* set by a worker that could not allocate */
    int64_t bh;              /* flat query head (for the dropout mask) */
    const dropout_cfg* drop; /* NULL: no dropout */
} bwd_ctx;

/* rows i: P_i, O_i, L_i, D_i, dS_i and dQ_i */
static void bwd_rows(void* p, int64_t begin, int64_t end) {
    bwd_ctx* c = (bwd_ctx*)p;
    const int64_t N = c->N, d = c->d;
    for (int64_t i = begin; i < end; ++i) {
        const double* qi = c->q + i * d;
        double* Pi = c->P + i * N;
        double* dSi = c->dS + i * N;
        double m = -INFINITY;
        for (int64_t j = 0; j < N; ++j) {
            Pi[j] = -INFINITY;
            if (!visible(c->causal, i, j)) continue;
            double dot = 0.0;
            for (int64_t t = 0; t < d; ++t) dot += qi[t] * c->k[j * d + t];
            Pi[j] = c->scale * dot; /* holds S_ij for now */
            if (Pi[j] > m) m = Pi[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < N; ++j)
            if (visible(c->causal, i, j)) l += exp(Pi[j] - m);
        for (int64_t j = 0; j < N; ++j)
            Pi[j] = (m == -INFINITY || !visible(c->causal, i, j)) ? 0.0 : exp(Pi[j] - m) / l;
        c->lse[i] = (m == -INFINITY) ? -INFINITY : m + log(l);
        /* Dropout factors z_ij (0 or the keep scale; 1 without dropout), kept
         * in dS_i until dS is formed. */
        for (int64_t j = 0; j < N; ++j) dSi[j] = dropout_factor(c->drop, c->bh, i, j);
        /* O_i = (P_i * z_i) V and D_i = dO_i . O_i */
        double* oi = c->o + i * d;
        for (int64_t t = 0; t < d; ++t) oi[t] = 0.0;
        for (int64_t j = 0; j < N; ++j)
            for (int64_t t = 0; t < d; ++t) oi[t] += Pi[j] * dSi[j] * c->v[j * d + t];
        const double* doi = c->dout + i * d;
        double Di = 0.0;
        for (int64_t t = 0; t < d; ++t) Di += doi[t] * oi[t];
        c->delta[i] = Di;
        /* dP_ij = dO_i . v_j ; dS_ij = P_ij (z_ij dP_ij - D_i) ; dQ_i = scale sum_j dS_ij k_j;
         * P_i then becomes P_i * z_i, the weights of dV. */
        double* dqi = c->dq + i * d;
        for (int64_t t = 0; t < d; ++t) dqi[t] = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            double dP = 0.0;
            for (int64_t t = 0; t < d; ++t) dP += doi[t] * c->v[j * d + t];
            const double z = dSi[j];
            dSi[j] = Pi[j] * (z * dP - Di);
            Pi[j] *= z;
            for (int64_t t = 0; t < d; ++t) dqi[t] += dSi[j] * c->k[j * d + t];
        }
        for (int64_t t = 0; t < d; ++t) dqi[t] *= c->scale;
    }
}

/* columns j: dV_j += sum_i (P z)_ij dO_i ; dK_j += scale sum_i dS_ij q_i (added to
 * what dv, dk hold: the key/value head may be shared by several query heads) */
static void bwd_cols(void* p, int64_t begin, int64_t end) {
    bwd_ctx* c = (bwd_ctx*)p;
    const int64_t N = c->N, d = c->d;
    double* sv = (double*)malloc(sizeof(double) * (size_t)(2 * d));
    if (!sv) {
        c->failed = 1;
        return;
    }
    double* sk = sv + d;
    for (int64_t j = begin; j < end; ++j) {
        double* dvj = c->dv + j * d;
        double* dkj = c->dk + j * d;
        for (int64_t t = 0; t < d; ++t) sv[t] = sk[t] = 0.0;
        /* each sum runs over i in increasing order */
        for (int64_t i = 0; i < N; ++i) {
            const double pij = c->P[i * N + j], dsij = c->dS[i * N + j];
            for (int64_t t = 0; t < d; ++t) {
                sv[t] += pij * c->dout[i * d + t];
                sk[t] += dsij * c->q[i * d + t];
            }
        }
        for (int64_t t = 0; t < d; ++t) {
            dvj[t] += sv[t];
            dkj[t] += c->scale * sk[t];
        }
    }
    free(sv);
}

/* delta may be NULL; otherwise it receives D = rowsum(dO * O) with the
 * oracle's own fp64 O. */
static int bwd_grouped(const double* q, const double* k, const double* v, const double* dout,
                       double* dq, double* dk, double* dv, double* delta, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t N, int64_t d, double scale, int causal, int nthreads,
                       const dropout_cfg* drop);

int oracle_attn_bwd(const double* q, const double* k, const double* v, const double* dout,
                    double* dq, double* dk, double* dv, double* delta,
                    int64_t BH, int64_t N, int64_t d, double scale, int causal, int nthreads) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv || BH <= 0 || N <= 0 || d <= 0)
        return ORACLE_ERR_ARG;
    return bwd_grouped(q, k, v, dout, dq, dk, dv, delta, 1, BH, BH, N, d, scale, causal, nthreads, NULL);
}

/* Grouped-head backward: q, dout, dq [B, Hq, N, d], delta [B, Hq, N],
 * k, v, dk, dv [B, Hkv, N, d], Hq a multiple of Hkv.  dk, dv are the sums
 * over the query heads sharing each key/value head. */
int oracle_attn_bwd_gqa(const double* q, const double* k, const double* v, const double* dout,
                        double* dq, double* dk, double* dv, double* delta, int64_t B, int64_t Hq,
                        int64_t Hkv, int64_t N, int64_t d, double scale, int causal, int nthreads) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv || B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 ||
        d <= 0 || Hq % Hkv != 0)
        return ORACLE_ERR_ARG;
    return bwd_grouped(q, k, v, dout, dq, dk, dv, delta, B, Hq, Hkv, N, d, scale, causal, nthreads, NULL);
}

/* Grouped-head backward with dropout of probability p (the mask of the
 * forward with the same seed and offset). */
int oracle_attn_bwd_dropout(const double* q, const double* k, const double* v, const double* dout, double* dq,
                            double* dk, double* dv, double* delta, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                            int64_t d, double scale, int causal, double p, uint64_t seed, uint64_t offset,
                            int nthreads) {
    dropout_cfg dc;
    if (!q || !k || !v || !dout || !dq || !dk || !dv || B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0 ||
        Hq % Hkv != 0 || dropout_setup(&dc, p, seed, offset) != ORACLE_OK)
        return ORACLE_ERR_ARG;
    return bwd_grouped(q, k, v, dout, dq, dk, dv, delta, B, Hq, Hkv, N, d, scale, causal, nthreads, &dc);
}

static int bwd_grouped(const double* q, const double* k, const double* v, const double* dout,
                       double* dq, double* dk, double* dv, double* delta, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t N, int64_t d, double scale, int causal, int nthreads,
                       const dropout_cfg* drop) {
    const int64_t BH = B * Hq, group = Hq / Hkv;
    double* P = (double*)malloc(sizeof(double) * (size_t)(N * N));
    double* dS = (double*)malloc(sizeof(double) * (size_t)(N * N));
    double* o = (double*)malloc(sizeof(double) * (size_t)(N * d));
    double* lse = (double*)malloc(sizeof(double) * (size_t)N);
    double* dl = (double*)malloc(sizeof(double) * (size_t)N);
    int rc = ORACLE_OK;
    if (!P || !dS || !o || !lse || !dl) rc = ORACLE_ERR_NOMEM;
    memset(dk, 0, sizeof(double) * (size_t)(B * Hkv * N * d));
    memset(dv, 0, sizeof(double) * (size_t)(B * Hkv * N * d));
    for (int64_t bh = 0; bh < BH && rc == ORACLE_OK; ++bh) {
        const int64_t off = bh * N * d, kvoff = kv_head(bh, Hq, group) * N * d;
        bwd_ctx c = {q + off, k + kvoff, v + kvoff, dout + off, dq + off, dk + kvoff, dv + kvoff, dl,
                     P, dS, o, lse, N, d, scale, causal, 0, bh, drop};
        rc = parallel_for(N, nthreads, bwd_rows, &c);
        if (rc == ORACLE_OK) rc = parallel_for(N, nthreads, bwd_cols, &c);
        if (rc == ORACLE_OK && c.failed) rc = ORACLE_ERR_NOMEM;
        if (delta) memcpy(delta + bh * N, dl, sizeof(double) * (size_t)N);
    }
    free(P);
    free(dS);
    free(o);
    free(lse);
    free(dl);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Tiled forward, in fp64: the keys are cut into blocks of bc, every block   */
/* is reduced on its own to a summary of each query row, and the summaries   */
/* are folded together with the online-softmax rescaling rule ("FlashAttention"
 * deep-dive page, "How it works": running maximum, running sum, rescale by   */
/* exp(m_old - m_new), one division at the end; the split-KV merge of its     */
/* "Implementation notes" is the same rule).                                  */
/*                                                                           */
/* Summary of key block b for query row i (visible keys only):               */
/*   mb = max_j s_ij,  lb = sum_j exp(s_ij - mb),  ab = sum_j exp(s_ij - mb) v_j */
/* Folding (mb, lb, ab) into the row's running (M, Lam, A):                   */
/*   M' = max(M, mb),  Lam' = exp(M - M') Lam + exp(mb - M') lb,              */
/*   A' = exp(M - M') A + exp(mb - M') ab                                     */
/* (a block with no visible key leaves the state as it is; the first block    */
/* that has one sets it).  At the end O_i = A / Lam and L_i = M + ln Lam.     */
/* Query rows are handled in groups of br; with exact arithmetic neither br   */
/* nor bc changes the result.                                                 */
/*                                                                           */
/* trace (may be NULL) receives, for query row trace_row of head 0, the      */
/* running state after each key block as 2 + d doubles: M, Lam, A[0..d-1].   */
/* It must hold ceil(N / bc) records.                                        */

typedef struct {
    double mx, sum; /* block maximum (-inf: nothing visible) and sum of exp(s - mx) */
    double* wv;     /* d values: sum of exp(s - mx) v_j */
} block_summary;

/* Summary of keys [j0, j1) of one head for query row i (q_row = Q_i). */
static void summarise_block(const double* q_row, const double* kh, const double* vh, int64_t d, double scale,
                            int causal, int64_t i, int64_t j0, int64_t j1, double* s_buf, block_summary* out) {
    out->mx = -INFINITY;
    for (int64_t j = j0; j < j1; ++j) {
        s_buf[j - j0] = -INFINITY;
        if (!visible(causal, i, j)) continue;
        double dot = 0.0;
        for (int64_t t = 0; t < d; ++t) dot += q_row[t] * kh[j * d + t];
        s_buf[j - j0] = scale * dot;
        if (s_buf[j - j0] > out->mx) out->mx = s_buf[j - j0];
    }
    out->sum = 0.0;
    for (int64_t t = 0; t < d; ++t) out->wv[t] = 0.0;
    if (out->mx == -INFINITY) return;
    for (int64_t j = j0; j < j1; ++j) {
        const double w = exp(s_buf[j - j0] - out->mx); /* exp(-inf) = 0 for masked keys */
        out->sum += w;
        for (int64_t t = 0; t < d; ++t) out->wv[t] += w * vh[j * d + t];
    }
}

/* Fold a block summary into a running state (M, Lam, A). */
static void fold_block(double* M, double* Lam, double* A, const block_summary* b, int64_t d) {
    if (b->mx == -INFINITY) return;
    if (*M == -INFINITY) {
        *M = b->mx;
        *Lam = b->sum;
        for (int64_t t = 0; t < d; ++t) A[t] = b->wv[t];
        return;
    }
    const double top = *M > b->mx ? *M : b->mx;
    const double w_run = exp(*M - top), w_blk = exp(b->mx - top);
    *Lam = w_run * *Lam + w_blk * b->sum;
    for (int64_t t = 0; t < d; ++t) A[t] = w_run * A[t] + w_blk * b->wv[t];
    *M = top;
}

int oracle_attn_fwd_tiled(const double* q, const double* k, const double* v, double* o, double* lse,
                          int64_t BH, int64_t N, int64_t d, double scale, int causal,
                          int64_t br, int64_t bc, int64_t trace_row, double* trace) {
    if (!q || !k || !v || !o || !lse || BH <= 0 || N <= 0 || d <= 0 || br <= 0 || bc <= 0)
        return ORACLE_ERR_ARG;
    /* running state of br rows: M[br], Lam[br], A[br * d]; one block summary */
    double* M = (double*)malloc(sizeof(double) * (size_t)br);
    double* Lam = (double*)malloc(sizeof(double) * (size_t)br);
    double* A = (double*)malloc(sizeof(double) * (size_t)(br * d));
    double* s_buf = (double*)malloc(sizeof(double) * (size_t)bc);
    double* wv = (double*)malloc(sizeof(double) * (size_t)d);
    int rc = ORACLE_OK;
    if (!M || !Lam || !A || !s_buf || !wv) rc = ORACLE_ERR_NOMEM;
    block_summary blk = {0.0, 0.0, wv};
    for (int64_t bh = 0; bh < BH && rc == ORACLE_OK; ++bh) {
        const double* qh = q + bh * N * d;
        const double* kh = k + bh * N * d;
        const double* vh = v + bh * N * d;
        for (int64_t g0 = 0; g0 < N; g0 += br) {
            const int64_t g1 = g0 + br < N ? g0 + br : N;
            for (int64_t i = g0; i < g1; ++i) {
                M[i - g0] = -INFINITY;
                Lam[i - g0] = 0.0;
                for (int64_t t = 0; t < d; ++t) A[(i - g0) * d + t] = 0.0;
            }
            for (int64_t b = 0; b * bc < N; ++b) {
                const int64_t j0 = b * bc, j1 = j0 + bc < N ? j0 + bc : N;
                for (int64_t i = g0; i < g1; ++i) {
                    double* Ai = A + (i - g0) * d;
                    summarise_block(qh + i * d, kh, vh, d, scale, causal, i, j0, j1, s_buf, &blk);
                    fold_block(&M[i - g0], &Lam[i - g0], Ai, &blk, d);
                    if (trace && bh == 0 && i == trace_row) {
                        double* rec = trace + b * (2 + d);
                        rec[0] = M[i - g0];
                        rec[1] = Lam[i - g0];
                        for (int64_t t = 0; t < d; ++t) rec[2 + t] = Ai[t];
                    }
                }
            }
            for (int64_t i = g0; i < g1; ++i) {
                double* oi = o + (bh * N + i) * d;
                const double* Ai = A + (i - g0) * d;
                const int none = M[i - g0] == -INFINITY; /* no visible key: O = 0, L = -inf */
                for (int64_t t = 0; t < d; ++t) oi[t] = none ? 0.0 : Ai[t] / Lam[i - g0];
                lse[bh * N + i] = none ? -INFINITY : M[i - g0] + log(Lam[i - g0]);
            }
        }
    }
    free(M);
    free(Lam);
    free(A);
    free(s_buf);
    free(wv);
    return rc;
}

int oracle_default_threads(void) { return resolve_threads(0); }
