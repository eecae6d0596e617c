/*
 * Plain CPU oracle for sparse (top-k index) MLA decode over a paged latent
 * cache.
 *
 * TEST INFRASTRUCTURE ONLY, under the same rules as mla_oracle.c: nothing in
 * the library or its binding may call, link or load it; it shares no code,
 * header or constant with the HIP path (nor with mla_oracle.c: it is written
 * out on its own so that each file can be checked by itself).
 *
 * What it computes: the same scaled dot-product attention of a new query
 * over cached latent rows as the dense decode (FlashMLA explainer,
 * theflyingbirds.in, section 4.1.1; "OpenSourceWeek Day 1: FlashMLA",
 * bibleofai.com, "How KV Caching Works?" and "How MLA Optimizes Memory
 * Usage?"; paged rows through the block table: same page, "Key Highlights",
 * explainer 4.3.2), but over a chosen subset of the cached tokens instead of
 * all of them: the dynamic sparse attention of DeepSeek v3.2 named on the
 * "Boosting DeepSeek V3.2" page (leadinhealth.com), where an indexer picks,
 * for each new token, which cached tokens it attends to.
 *
 * Readings where the pages are silent (listed in the design notes):
 *   - the list of new token i of sequence b is indices[b][i][0 .. n) with
 *     n = counts[b * s_q + i]; all heads of that token share it;
 *   - entries < 0 are padding and are skipped; any other entry t is a token
 *     position of sequence b (row t % page of block block_table[b][t / page]);
 *     a repeated position counts once per occurrence;
 *   - no causal mask beyond the list itself; a list with no valid entry
 *     gives out = 0 and lse = -inf; lse is the natural log and includes the
 *     scale.
 *
 * Arithmetic: bf16 inputs widened exactly, every product, sum, exp and log in
 * double precision, one query row at a time, tokens in list order.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const uint16_t* q;             /* [B, s_q, h_q, d_qk] bf16 bits */
    const uint16_t* kcache;        /* [nblocks, page, d_qk] */
    const int32_t* block_table;    /* [B, max_blocks] */
    const int32_t* indices;        /* [B, s_q, topk] */
    const int32_t* counts;         /* [B * s_q] */
    int B, s_q, h_q, max_blocks, topk, d_qk, d_v, page;
    double scale;
    double* out;                   /* [B, s_q, h_q, d_v] */
    double* lse;                   /* [B, s_q, h_q] */
    int nthreads, thread_id, status;
} sparse_job;

static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int sparse_row(const sparse_job* a, int b, int i, int h)
{
    const long row = ((long)b * a->s_q + i) * a->h_q + h;
    const uint16_t* qrow = a->q + row * (long)a->d_qk;
    const int32_t* list = a->indices + ((long)b * a->s_q + i) * a->topk;
    const int n = a->counts[(long)b * a->s_q + i];
    double* out = a->out + row * (long)a->d_v;
    for (int c = 0; c < a->d_v; ++c) out[c] = 0.0;

    const uint16_t** rows = (const uint16_t**)malloc(sizeof(uint16_t*) * (size_t)(n > 0 ? n : 1));
    double* score = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!rows || !score) { free(rows); free(score); return -1; }
    int used = 0;
    for (int k = 0; k < n; ++k) {
        const long t = list[k];
        if (t < 0) continue;
        const long blk = a->block_table[(long)b * a->max_blocks + t / a->page];
        rows[used++] = a->kcache + (blk * a->page + t % a->page) * (long)a->d_qk;
    }
    if (used == 0) {
        a->lse[row] = -INFINITY;
        free(rows); free(score);
        return 0;
    }
    for (int u = 0; u < used; ++u) {
        double dot = 0.0;
        for (int d = 0; d < a->d_qk; ++d) dot += widen_bf16(qrow[d]) * widen_bf16(rows[u][d]);
        score[u] = a->scale * dot;
    }
    double m = score[0];
    for (int u = 1; u < used; ++u) m = score[u] > m ? score[u] : m;
    double z = 0.0;
    for (int u = 0; u < used; ++u) z += exp(score[u] - m);
    for (int u = 0; u < used; ++u) {
        const double w = exp(score[u] - m) / z;
        for (int c = 0; c < a->d_v; ++c) out[c] += w * widen_bf16(rows[u][c]);
    }
    a->lse[row] = m + log(z);
    free(rows); free(score);
    return 0;
}

static void* sparse_worker(void* p)
{
    sparse_job* a = (sparse_job*)p;
    const long nrows = (long)a->B * a->s_q * a->h_q;
    for (long r = a->thread_id; r < nrows; r += a->nthreads) {
        const int h = (int)(r % a->h_q);
        const int i = (int)((r / a->h_q) % a->s_q);
        const int b = (int)(r / ((long)a->h_q * a->s_q));
        if (sparse_row(a, b, i, h) != 0) { a->status = -1; return NULL; }
    }
    return NULL;
}

/*
 * Sparse decode attention of every query row over its token list.
 * Returns 0, or -1 on bad arguments or allocation failure. The caller
 * guarantees 0 <= counts[.] <= topk and that every listed token's block-table
 * entry is a valid block.
 */
int mla_oracle_decode_sparse(const uint16_t* q, const uint16_t* kcache, const int32_t* block_table,
                             const int32_t* indices, const int32_t* counts, int B, int s_q, int h_q,
                             int max_blocks, int topk, int d_qk, int d_v, int page, double softmax_scale,
                             double* out, double* lse, int nthreads)
{
    if (B < 0 || s_q < 1 || h_q < 1 || topk < 1 || d_qk < 1 || d_v < 1 || d_v > d_qk || page < 1) return -1;
    if (B == 0) return 0;
    if (!q || !kcache || !block_table || !indices || !counts || !out || !lse) return -1;
    for (long k = 0; k < (long)B * s_q; ++k)
        if (counts[k] < 0 || counts[k] > topk) return -1;
    if (nthreads < 1) nthreads = 1;
    sparse_job base;
    memset(&base, 0, sizeof base);
    base.q = q; base.kcache = kcache; base.block_table = block_table; base.indices = indices;
    base.counts = counts; base.B = B; base.s_q = s_q; base.h_q = h_q; base.max_blocks = max_blocks;
    base.topk = topk; base.d_qk = d_qk; base.d_v = d_v; base.page = page; base.scale = softmax_scale;
    base.out = out; base.lse = lse; base.nthreads = nthreads;
    sparse_job* jobs = (sparse_job*)malloc(sizeof(sparse_job) * (size_t)nthreads);
    pthread_t* tids = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!jobs || !tids) { free(jobs); free(tids); return -1; }
    for (int k = 0; k < nthreads; ++k) {
        jobs[k] = base;
        jobs[k].thread_id = k;
        if (k > 0 && pthread_create(&tids[k], NULL, sparse_worker, &jobs[k]) != 0) jobs[k].status = -2;
    }
    sparse_worker(&jobs[0]);
    int status = jobs[0].status;
    for (int k = 1; k < nthreads; ++k) {
        if (jobs[k].status == -2) {
            jobs[k].status = 0;
            sparse_worker(&jobs[k]);
        } else {
            pthread_join(tids[k], NULL);
        }
        if (jobs[k].status != 0) status = -1;
    }
    free(jobs);
    free(tids);
    return status;
}
