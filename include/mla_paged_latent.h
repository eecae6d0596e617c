/*
 * mla_paged_latent.h -- C ABI of the MI355X (gfx950) library for Multi-head
 * Latent Attention decoding over a paged, compressed latent KV cache.
 *
 * The operation (what the library computes):
 *   For every sequence b, new-token position i and query head h,
 *     out[b,i,h,:] = sum_t softmax_t(scale * q[b,i,h,:] . k_t) * k_t[0:512]
 *     lse[b,i,h]   = ln sum_t exp(scale * q[b,i,h,:] . k_t)
 *   over the cached rows k_t (576 bf16 each) that the query sees.
 *   - Scaled dot-product attention: FlashMLA explainer (theflyingbirds.in),
 *     section 4.1.1 "Mathematical Formulation".
 *   - Decode: only the new queries are computed; they attend over the
 *     cached entries: "OpenSourceWeek Day 1: FlashMLA" (bibleofai.com),
 *     section "How KV Caching Works?".
 *   - MLA caches one latent row per token, shared by all heads; keys and
 *     values are linear maps of it: same page, "How MLA Optimizes Memory
 *     Usage?". With those maps folded into q and applied to out by the
 *     caller, the score uses all 576 cached columns (512 latent + 64 rope)
 *     and the value is the first 512 columns of the same row.
 *   - Paged cache, block size 64, BF16: same page, "Key Highlights";
 *     explainer section 4.3.2 "Paged KV Cache".
 *   - Variable-length batches: GeekNews release note (id.news.hada.io).
 *   Readings where the pages say nothing:
 *   - the s_q new tokens are the last s_q cached positions of their
 *     sequence (cache_seqlens counts them); with causal != 0, query i
 *     (0-based) sees tokens [0, L - s_q + i], otherwise [0, L);
 *   - lse is the natural log and includes the scale;
 *   - a query that sees no token gets out = 0 and lse = -inf.
 *
 * Conventions for every call:
 *   - Device pointers point to memory on the current HIP device; the caller
 *     owns every buffer. The library allocates nothing, frees nothing and
 *     keeps no pointer after a call returns.
 *   - `stream` is a hipStream_t (NULL = the null stream). Device calls only
 *     enqueue work on it: no host synchronisation, no device-to-host copy.
 *   - Arguments are checked on the host before anything is enqueued; a
 *     failed check returns a negative mla_status and enqueues nothing.
 *     A failed launch returns MLA_ERR_HIP.
 *   - Contracts the host cannot check (undefined behaviour if broken):
 *     0 <= cache_seqlens[b] <= 64 * max_blocks, and block_table[b][j] is in
 *     [0, nblocks) for every j < ceil(cache_seqlens[b] / 64). Other table
 *     entries are never read, and cache rows at or past cache_seqlens[b]
 *     never influence a result (they may hold anything, NaN included).
 */
#ifndef MLA_PAGED_LATENT_H
#define MLA_PAGED_LATENT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_D_QK 576            /* cached row width: 512 latent + 64 rope columns */
#define MLA_D_V 512             /* value width: the first 512 columns of a cached row */
#define MLA_PAGE_SIZE 64        /* tokens per cache block */
#define MLA_META_INTS 8         /* int32 entries per work unit in tile_meta */

typedef enum mla_status {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = -1,         /* null pointer, non-positive size, bad alignment */
    MLA_ERR_UNSUPPORTED = -2,         /* shape the kernels do not handle (s_q*h_q) */
    MLA_ERR_WORKSPACE_TOO_SMALL = -3,
    MLA_ERR_HIP = -4                  /* a HIP runtime call or launch failed */
} mla_status;

/* Human-readable text for a status code. Never NULL. */
const char* mla_status_string(int status);

/*
 * Host-only sizing for the buffers the caller allocates.
 *   batch, s_q, h_q: as for mla_decode_fwd. s_q*h_q must be a multiple of 16
 *     in [16, 1024].
 *   num_cus: compute units to plan for; <= 0 asks the current HIP device.
 * Outputs (any may be NULL):
 *   num_units: work units the plan splits the batch into (pass it to both calls);
 *   meta_bytes: bytes of tile_meta (int32 [num_units, MLA_META_INTS]);
 *   splits_bytes: bytes of num_splits (int32 [batch + 1]);
 *   workspace_bytes: bytes of the split-KV workspace mla_decode_fwd needs.
 * Errors: MLA_ERR_INVALID_ARG (batch < 1, s_q < 1, h_q < 1),
 *   MLA_ERR_UNSUPPORTED (s_q*h_q), MLA_ERR_HIP (device query failed).
 */
int mla_plan_sizes(int batch, int s_q, int h_q, int num_cus, int* num_units,
                   size_t* meta_bytes, size_t* splits_bytes, size_t* workspace_bytes);

/*
 * Host-only: workspace bytes mla_decode_fwd needs for a plan of num_units
 * units (the value mla_plan_sizes reports for its own num_units).
 * Errors: MLA_ERR_INVALID_ARG (bad sizes, NULL output), MLA_ERR_UNSUPPORTED.
 */
int mla_workspace_bytes(int batch, int s_q, int h_q, int num_units, size_t* workspace_bytes);

/*
 * Split-KV tile plan for a variable-length batch (the pages only say the
 * kernel is tuned for variable-length serving: GeekNews release note).
 * Each unit is one workgroup's run of cache blocks, contiguous in (sequence,
 * block) order; every block belongs to exactly one unit. When s_q*h_q is a
 * multiple of 64 the blocks, with a fixed extra cost per sequence, are cut
 * into num_units runs of near-equal cost (a run may span sequences);
 * otherwise each sequence is cut into near-equal runs of at most
 * ceil(total_blocks / (num_units - batch)) blocks, and num_units must be at
 * least batch + 1.
 *   cache_seqlens: device int32 [batch].
 *   tile_meta: device int32 [num_units, MLA_META_INTS], written. Row u is
 *     {b_begin, blk_begin, b_end, blk_end, split_index, L, slot, nsplit}:
 *     unit u covers blocks (b, j) with (b_begin, blk_begin) <= (b, j) <
 *     (b_end, blk_end) in lexicographic order, j < ceil(L_b/64); split_index
 *     is how many earlier units touch sequence b_begin; L = cache_seqlens
 *     [b_begin], slot = num_splits[b_begin] + split_index and nsplit = the
 *     number of units touching b_begin (all three 0 for an empty unit).
 *   num_splits: device int32 [batch + 1], written: exclusive prefix sums of
 *     the number of units touching each sequence (0 for an empty sequence).
 * One small kernel on `stream`. The plan depends only on cache_seqlens,
 * batch, s_q, h_q and num_units, so one plan serves every layer of a step.
 */
int mla_get_metadata(const int32_t* cache_seqlens, int batch, int s_q, int h_q, int num_units,
                     int32_t* tile_meta, int32_t* num_splits, void* stream);

/*
 * The same plan computed on the host from host arrays (bit-identical to
 * mla_get_metadata). No HIP call. For tests and for callers that plan on
 * the CPU.
 */
int mla_get_metadata_host(const int32_t* cache_seqlens, int batch, int s_q, int h_q, int num_units,
                          int32_t* tile_meta, int32_t* num_splits);

/*
 * Decode attention over the paged latent cache.
 *   q: device bf16 [batch, s_q, h_q, 576], contiguous, 16-byte aligned.
 *   kcache: device bf16 [nblocks, 64, 576], contiguous, 16-byte aligned.
 *   block_table: device int32 [batch, max_blocks], row-major.
 *   cache_seqlens: device int32 [batch], cached tokens per sequence
 *     including the s_q new ones.
 *   softmax_scale: multiplies q.k before the softmax (finite).
 *   causal: nonzero masks, for query i, tokens past L - s_q + i.
 *   tile_meta, num_splits, num_units: a plan from mla_get_metadata for the
 *     same cache_seqlens, batch, s_q and h_q.
 *   out: device bf16 [batch, s_q, h_q, 512], written (round to nearest even).
 *   lse: device float [batch, s_q, h_q], written.
 *   workspace: device memory of at least the size mla_plan_sizes reports,
 *     16-byte aligned; its contents on entry do not matter.
 * Enqueues the decode kernel and the split combine kernel on `stream`.
 * Calls that share a workspace must not overlap in time.
 * Errors: MLA_ERR_INVALID_ARG (null or misaligned pointer, batch < 1,
 *   nblocks < 1, max_blocks < 1, num_units too small for the plan shape,
 *   non-finite scale),
 *   MLA_ERR_UNSUPPORTED (s_q*h_q), MLA_ERR_WORKSPACE_TOO_SMALL, MLA_ERR_HIP.
 */
int mla_decode_fwd(const void* q, const void* kcache, int64_t nblocks,
                   const int32_t* block_table, int max_blocks,
                   const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                   float softmax_scale, int causal,
                   const int32_t* tile_meta, const int32_t* num_splits, int num_units,
                   void* out, float* lse, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * The two stages of mla_decode_fwd as separate calls (same arguments and
 * checks), for callers that time or schedule the two kernels apart:
 * mla_decode_fwd is exactly mla_decode_fwd_splits followed by
 * mla_combine_splits on the same stream with the same workspace.
 * mla_decode_fwd_splits writes out/lse of sequences the plan did not split
 * and leaves fp32 partial results of split ones in the workspace;
 * mla_combine_splits merges those partials by their log-sum-exp (and writes
 * out = 0, lse = -inf for sequences with no cached token).
 */
int mla_decode_fwd_splits(const void* q, const void* kcache, int64_t nblocks,
                          const int32_t* block_table, int max_blocks,
                          const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                          float softmax_scale, int causal,
                          const int32_t* tile_meta, const int32_t* num_splits, int num_units,
                          void* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream);

int mla_combine_splits(const int32_t* num_splits, int batch, int s_q, int h_q, int num_units,
                       void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PAGED_LATENT_H */
