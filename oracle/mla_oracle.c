/*
 * Plain CPU oracle for MLA decode over a paged latent cache.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library or its Python binding may
 * call, link or load this file; only the tests, the smoke check and the
 * benchmark's CPU-baseline leg do. It shares no code, header or constant with
 * the HIP path.
 *
 * What it computes (one query row at a time, no tiling, no reordering):
 *
 *   Attention(Q, K, V) = softmax(Q K^T * scale) V
 *     -- FlashMLA explainer (theflyingbirds.in), section 4.1.1,
 *        "Mathematical Formulation", the attention-score formula.
 *
 *   Only the new query is computed at a decode step; it attends over the
 *   key/value entries already held in the cache
 *     -- "OpenSourceWeek Day 1: FlashMLA" (bibleofai.com), section
 *        "How KV Caching Works?".
 *
 *   MLA caches one latent vector c_t per token instead of per-head K and V;
 *   per-head keys and values are linear maps of c_t
 *     -- same page, section "How MLA Optimizes Memory Usage?".
 *   With the up-projections folded into the query (and applied to the output
 *   afterwards, outside this operation), every head attends directly over
 *   the shared cached rows: the score uses all d_qk columns of a row and the
 *   value is its first d_v columns.
 *
 *   The cache is paged: a sequence's tokens live in fixed blocks of `page`
 *   rows that need not be contiguous, found through a block table
 *     -- same page, "Key Highlights" (block size 64); explainer section
 *        4.3.2 "Paged KV Cache" (virtual-memory analogy).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - s_q new tokens per sequence are the last s_q cached positions; with
 *     causal=1 query i (0-based) sees tokens [0, L - s_q + i], else [0, L).
 *   - lse = natural log of sum_t exp(scale * q.k_t).
 *   - a row that sees no token gets out = 0 and lse = -inf.
 *
 * Arithmetic: inputs are bf16 bit patterns, widened exactly; every product,
 * sum, exp and log is done in double precision. Results are double.
 *
 * Parity pins: tests/test_oracle_pins.py checks this file against a library
 * attention routine, closed forms (one visible token, equal scores, weights
 * fixed by the scale), exact invariances (block-table permutation, causal
 * prefix), the two-part log-sum-exp merge, NaN-poisoned unread rows, and a
 * set of planted mistakes that those checks must catch.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const uint16_t* q;             /* [B, s_q, h_q, d_qk] bf16 bits */
    const uint16_t* kcache;        /* [nblocks, page, d_qk] bf16 bits */
    const int32_t* block_table;    /* [B, max_blocks] */
    const int32_t* cache_seqlens;  /* [B] */
    int B, s_q, h_q, max_blocks, d_qk, d_v, page, causal;
    double scale;
    double* out;                   /* [B, s_q, h_q, d_v] */
    double* lse;                   /* [B, s_q, h_q] */
    int nthreads;
    int thread_id;
    int status;
} oracle_job;

static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* The cached row holding token t of sequence b. */
static const uint16_t* cached_row(const oracle_job* a, int b, long t)
{
    long j = t / a->page;
    long r = t % a->page;
    long phys = a->block_table[(long)b * a->max_blocks + j];
    return a->kcache + (phys * a->page + r) * (long)a->d_qk;
}

/* One query row (b, i, h): scores over every visible token, softmax, weighted
 * sum of the value columns. Returns 0, or -1 if scratch memory ran out. */
static int attend_one_row(const oracle_job* a, int b, int i, int h)
{
    const long row = ((long)b * a->s_q + i) * a->h_q + h;
    const uint16_t* qrow = a->q + row * (long)a->d_qk;
    double* out = a->out + row * (long)a->d_v;
    long L = a->cache_seqlens[b];
    long visible = a->causal ? L - (a->s_q - 1 - i) : L;

    for (int c = 0; c < a->d_v; ++c) out[c] = 0.0;
    if (visible <= 0) {
        a->lse[row] = -INFINITY;
        return 0;
    }

    double* score = (double*)malloc(sizeof(double) * (size_t)visible);
    if (!score) return -1;

    /* s_t = scale * sum_d q[d] * k_t[d] over all d_qk columns */
    for (long t = 0; t < visible; ++t) {
        const uint16_t* k = cached_row(a, b, t);
        double dot = 0.0;
        for (int d = 0; d < a->d_qk; ++d) dot += bf16_value(qrow[d]) * bf16_value(k[d]);
        score[t] = a->scale * dot;
    }

    /* softmax with the maximum taken out first, so exp never overflows */
    double m = score[0];
    for (long t = 1; t < visible; ++t)
        if (score[t] > m) m = score[t];
    double denom = 0.0;
    for (long t = 0; t < visible; ++t) denom += exp(score[t] - m);

    /* out = sum_t softmax_t * v_t, v_t = first d_v columns of the cached row */
    for (long t = 0; t < visible; ++t) {
        const uint16_t* v = cached_row(a, b, t);
        double w = exp(score[t] - m) / denom;
        for (int c = 0; c < a->d_v; ++c) out[c] += w * bf16_value(v[c]);
    }
    a->lse[row] = m + log(denom);
    free(score);
    return 0;
}

static void* worker(void* p)
{
    oracle_job* a = (oracle_job*)p;
    const long rows = (long)a->B * a->s_q * a->h_q;
    for (long r = a->thread_id; r < rows; r += a->nthreads) {
        int h = (int)(r % a->h_q);
        int i = (int)((r / a->h_q) % a->s_q);
        int b = (int)(r / ((long)a->h_q * a->s_q));
        if (attend_one_row(a, b, i, h) != 0) {
            a->status = -1;
            return NULL;
        }
    }
    return NULL;
}

/*
 * Decode attention of every query row over its sequence's paged cache.
 * Returns 0 on success, -1 on bad arguments or allocation failure.
 * The caller guarantees block_table[b][j] is a valid block for every
 * j < ceil(cache_seqlens[b] / page); other entries are never read.
 */
int mla_oracle_decode(const uint16_t* q, const uint16_t* kcache, const int32_t* block_table,
                      const int32_t* cache_seqlens, int B, int s_q, int h_q, int max_blocks,
                      int d_qk, int d_v, int page, double softmax_scale, int causal,
                      double* out, double* lse, int nthreads)
{
    if (B < 0 || s_q < 1 || h_q < 1 || d_qk < 1 || d_v < 1 || d_v > d_qk || page < 1) return -1;
    if (B == 0) return 0;
    if (!q || !kcache || !block_table || !cache_seqlens || !out || !lse) return -1;
    if (nthreads < 1) nthreads = 1;

    oracle_job base;
    base.q = q; base.kcache = kcache; base.block_table = block_table;
    base.cache_seqlens = cache_seqlens;
    base.B = B; base.s_q = s_q; base.h_q = h_q; base.max_blocks = max_blocks;
    base.d_qk = d_qk; base.d_v = d_v; base.page = page; base.causal = causal ? 1 : 0;
    base.scale = softmax_scale; base.out = out; base.lse = lse;
    base.nthreads = nthreads; base.status = 0;

    oracle_job* jobs = (oracle_job*)malloc(sizeof(oracle_job) * (size_t)nthreads);
    pthread_t* tids = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!jobs || !tids) { free(jobs); free(tids); return -1; }
    int started = 0;
    for (int k = 0; k < nthreads; ++k) {
        jobs[k] = base;
        jobs[k].thread_id = k;
        if (k == 0) continue;
        if (pthread_create(&tids[k], NULL, worker, &jobs[k]) != 0) { jobs[k].status = -2; continue; }
        ++started;
    }
    worker(&jobs[0]);
    int status = jobs[0].status;
    for (int k = 1; k < nthreads; ++k) {
        if (jobs[k].status == -2) {          /* thread never started: do its rows here */
            jobs[k].status = 0;
            worker(&jobs[k]);
        } else {
            pthread_join(tids[k], NULL);
        }
        if (jobs[k].status != 0) status = -1;
    }
    (void)started;
    free(jobs);
    free(tids);
    return status;
}
