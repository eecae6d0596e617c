/*
 * Plain CPU oracle for MLA decode over an FP8 paged latent cache.
 *
 * TEST INFRASTRUCTURE ONLY, under the same rules as mla_oracle.c: nothing in
 * the library or its binding may call, link or load it; it shares no code,
 * header or constant with the HIP path (nor with the other oracle files).
 *
 * What it computes: the decode attention of mla_oracle.c (FlashMLA explainer,
 * theflyingbirds.in, section 4.1.1; "OpenSourceWeek Day 1: FlashMLA",
 * bibleofai.com, "How KV Caching Works?", "How MLA Optimizes Memory Usage?",
 * "Key Highlights"; explainer 4.3.2 for the paging), over a cache whose rows
 * are stored in 8-bit floating point -- the FP8 support the FlashMLA
 * explainer lists under section 9, "Future Directions", to cut memory
 * further -- each row with one float32 scale:
 *   k_t[d] = e4m3(code_t[d]) * scale_t.
 * Readings where the pages are silent (listed in the design notes): the 8-bit
 * format is OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals, no infinities, 0x7F / 0xFF = NaN); one scale per cached row
 * covers all 576 columns; the query stays bf16 and the output is the same as
 * for a bf16 cache holding the decoded values.
 *
 * Arithmetic: every decoded value, product, sum, exp and log in double
 * precision, one query row at a time.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* E4M3 (OCP) from its definition. */
double mla_oracle_e4m3_value(uint8_t code)
{
    const int sign = code >> 7;
    const int expo = (code >> 3) & 15;
    const int mant = code & 7;
    double v;
    if (expo == 15 && mant == 7) return NAN;
    if (expo == 0) v = ldexp((double)mant / 8.0, -6);           /* subnormal: 0.mmm x 2^(1-7) */
    else v = ldexp(1.0 + (double)mant / 8.0, expo - 7);
    return sign ? -v : v;
}

typedef struct {
    const uint16_t* q;          /* [B, s_q, h_q, d_qk] bf16 bits */
    const uint8_t* codes;       /* [nblocks, page, d_qk] E4M3 */
    const float* scales;        /* [nblocks, page] */
    const int32_t* block_table; /* [B, max_blocks] */
    const int32_t* cache_seqlens;
    int B, s_q, h_q, max_blocks, d_qk, d_v, page, causal;
    double scale;
    double* out;
    double* lse;
    int nthreads, thread_id, status;
} fp8_job;

static double q_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int fp8_row(const fp8_job* a, int b, int i, int h)
{
    const long row = ((long)b * a->s_q + i) * a->h_q + h;
    const uint16_t* qrow = a->q + row * (long)a->d_qk;
    double* out = a->out + row * (long)a->d_v;
    const long L = a->cache_seqlens[b];
    const long n = a->causal ? L - (a->s_q - 1 - i) : L;
    for (int c = 0; c < a->d_v; ++c) out[c] = 0.0;
    if (n <= 0) {
        a->lse[row] = -INFINITY;
        return 0;
    }
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    if (!s) return -1;
    for (long t = 0; t < n; ++t) {
        const long phys = (long)a->block_table[(long)b * a->max_blocks + t / a->page] * a->page + t % a->page;
        const uint8_t* k = a->codes + phys * (long)a->d_qk;
        const double ks = (double)a->scales[phys];
        double dot = 0.0;
        for (int d = 0; d < a->d_qk; ++d) dot += q_value(qrow[d]) * (mla_oracle_e4m3_value(k[d]) * ks);
        s[t] = a->scale * dot;
    }
    double m = s[0];
    for (long t = 1; t < n; ++t) m = s[t] > m ? s[t] : m;
    double z = 0.0;
    for (long t = 0; t < n; ++t) z += exp(s[t] - m);
    for (long t = 0; t < n; ++t) {
        const long phys = (long)a->block_table[(long)b * a->max_blocks + t / a->page] * a->page + t % a->page;
        const uint8_t* v = a->codes + phys * (long)a->d_qk;
        const double vs = (double)a->scales[phys];
        const double w = exp(s[t] - m) / z;
        for (int c = 0; c < a->d_v; ++c) out[c] += w * (mla_oracle_e4m3_value(v[c]) * vs);
    }
    a->lse[row] = m + log(z);
    free(s);
    return 0;
}

static void* fp8_worker(void* p)
{
    fp8_job* a = (fp8_job*)p;
    const long nrows = (long)a->B * a->s_q * a->h_q;
    for (long r = a->thread_id; r < nrows; r += a->nthreads) {
        const int h = (int)(r % a->h_q);
        const int i = (int)((r / a->h_q) % a->s_q);
        const int b = (int)(r / ((long)a->h_q * a->s_q));
        if (fp8_row(a, b, i, h) != 0) { a->status = -1; return NULL; }
    }
    return NULL;
}

/* Decode over the FP8 cache. Returns 0, or -1 on bad arguments / allocation failure. */
int mla_oracle_decode_fp8(const uint16_t* q, const uint8_t* codes, const float* scales, const int32_t* block_table,
                          const int32_t* cache_seqlens, int B, int s_q, int h_q, int max_blocks, int d_qk, int d_v,
                          int page, double softmax_scale, int causal, double* out, double* lse, int nthreads)
{
    if (B < 0 || s_q < 1 || h_q < 1 || d_qk < 1 || d_v < 1 || d_v > d_qk || page < 1) return -1;
    if (B == 0) return 0;
    if (!q || !codes || !scales || !block_table || !cache_seqlens || !out || !lse) return -1;
    if (nthreads < 1) nthreads = 1;
    fp8_job base;
    memset(&base, 0, sizeof base);
    base.q = q; base.codes = codes; base.scales = scales; base.block_table = block_table;
    base.cache_seqlens = cache_seqlens; base.B = B; base.s_q = s_q; base.h_q = h_q;
    base.max_blocks = max_blocks; base.d_qk = d_qk; base.d_v = d_v; base.page = page;
    base.causal = causal ? 1 : 0; base.scale = softmax_scale; base.out = out; base.lse = lse;
    base.nthreads = nthreads;
    fp8_job* jobs = (fp8_job*)malloc(sizeof(fp8_job) * (size_t)nthreads);
    pthread_t* tids = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!jobs || !tids) { free(jobs); free(tids); return -1; }
    for (int k = 0; k < nthreads; ++k) {
        jobs[k] = base;
        jobs[k].thread_id = k;
        if (k > 0 && pthread_create(&tids[k], NULL, fp8_worker, &jobs[k]) != 0) jobs[k].status = -2;
    }
    fp8_worker(&jobs[0]);
    int status = jobs[0].status;
    for (int k = 1; k < nthreads; ++k) {
        if (jobs[k].status == -2) {
            jobs[k].status = 0;
            fp8_worker(&jobs[k]);
        } else {
            pthread_join(tids[k], NULL);
        }
        if (jobs[k].status != 0) status = -1;
    }
    free(jobs);
    free(tids);
    return status;
}
