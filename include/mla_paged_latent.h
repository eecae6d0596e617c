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
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)  /* device scratch of mla_decode_fwd_noalloc */

typedef enum mla_status {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = -1,         /* null pointer, non-positive size, bad alignment */
    MLA_ERR_UNSUPPORTED = -2,         /* shape the kernels do not handle (s_q*h_q) */
    MLA_ERR_WORKSPACE_TOO_SMALL = -3,
    MLA_ERR_HIP = -4,                 /* a HIP runtime call or launch failed */
    MLA_ERR_OUT_OF_BLOCKS = -5,       /* block pool: not enough free blocks (nothing changed) */
    MLA_ERR_OUT_OF_MEMORY = -6        /* block pool: host allocation failed (nothing changed) */
} mla_status;

/* Human-readable text for a status code. Never NULL. */
const char* mla_status_string(int status);

/*
 * Host-only sizing for the buffers the caller allocates.
 *   batch, s_q, h_q: as for mla_decode_fwd. s_q*h_q must be a multiple of 16
 *     in [16, 1024].
 *   num_cus: compute units to plan for; <= 0 asks the current HIP device.
 * Outputs (any may be NULL):
 *   num_units: work units the plan splits the batch into (pass it to both calls):
 *     num_cus / head groups for the 64-row kernels, (num_cus - num_cus / 8) /
 *     head groups but at least batch + 1 for the 16-row kernels;
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

/*
 * Host-only check of the contract the decode calls place on their device
 * inputs, on host copies of them: 0 <= cache_seqlens[b] <= 64 * max_blocks and
 * block_table[b][j] in [0, nblocks) for every j < ceil(cache_seqlens[b] / 64).
 * Returns MLA_OK, or MLA_ERR_INVALID_ARG with *bad_seq (if not NULL) set to the
 * first sequence that breaks it (-1 when all hold). No HIP call.
 * The decode kernels never read outside kcache or the table even when the
 * contract is broken (an entry outside [0, nblocks), or an index past the
 * table, reads block 0; the append calls skip such rows), but the results of
 * the sequences concerned are then unspecified. With the environment variable
 * MLA_DEBUG_CHECK set (and not "0"), mla_decode_fwd, mla_decode_fwd_splits,
 * mla_decode_fp8_fwd and mla_decode_fp8_fwd_splits copy cache_seqlens and
 * block_table to the host and apply this check before enqueueing anything
 * (synchronising; for debugging only).
 */
int mla_check_inputs_host(const int32_t* cache_seqlens, int batch, const int32_t* block_table, int max_blocks,
                          int64_t nblocks, int* bad_seq);

/*
 * mla_decode_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Arguments, results and checks are those
 * of mla_decode_fwd; the split partials go to a fixed device array of
 * MLA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends. The call allocates nothing and calls no
 * allocating routine; the first call on a device looks the array's address up
 * once (make that call outside a stream capture).
 * Limit: the workspace mla_workspace_bytes reports for (batch, s_q, h_q,
 *   num_units) must fit in MLA_NOALLOC_SCRATCH_BYTES, else
 *   MLA_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.
 * Every call on a GPU shares that GPU's array: calls that overlap in time on
 * one GPU (several streams, several host threads) race; serialise them.
 */
int mla_decode_fwd_noalloc(const void* q, const void* kcache, int64_t nblocks,
                           const int32_t* block_table, int max_blocks,
                           const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                           float softmax_scale, int causal,
                           const int32_t* tile_meta, const int32_t* num_splits, int num_units,
                           void* out, float* lse, void* stream);

/*
 * Sparse (top-k index) decode: each new token attends over its own list of
 * cached token positions instead of all of them -- the dynamic sparse
 * attention of DeepSeek v3.2 named on the "Boosting DeepSeek V3.2" page
 * (leadinhealth.com), an indexer choosing the tokens each query attends to.
 * The attention itself is that of mla_decode_fwd restricted to the listed
 * rows; all heads of a new token share its list. Readings where the pages are
 * silent: list entries < 0 are padding and skipped; a repeated position
 * counts once per occurrence; no causal mask beyond the list; a list with no
 * valid entry gives out = 0, lse = -inf.
 *
 * mla_sparse_plan_sizes: like mla_plan_sizes for a sparse batch (topk = the
 *   list capacity, 1..2048; h_q a multiple of 16 in [16, 1024]; batch*s_q
 *   lists at most 16384).
 * mla_get_metadata_sparse: the split plan of the batch*s_q lists (one small
 *   kernel on `stream`), from topk_lens: device int32 [batch*s_q], the number
 *   of leading list entries in use, 0..topk. tile_meta / num_splits as for
 *   mla_get_metadata with batch*s_q "sequences".
 * mla_decode_sparse_fwd: the decode. q, kcache, block_table, out, lse,
 *   workspace as for mla_decode_fwd; indices: device int32 [batch, s_q, topk],
 *   list of new token i of sequence b = indices[b][i][0 .. topk_lens[b*s_q+i]).
 *   Contracts the host cannot check: 0 <= topk_lens[.] <= topk; a listed
 *   position t has a valid block block_table[b][t / 64] (entries with t / 64
 *   >= max_blocks or a negative table entry are treated as padding).
 * mla_decode_sparse_fwd_splits: the decode kernel of mla_decode_sparse_fwd
 *   alone (same arguments and checks), as mla_decode_fwd_splits is for
 *   mla_decode_fwd: mla_decode_sparse_fwd is exactly it followed by
 *   mla_combine_splits(num_splits, batch * s_q, 1, h_q, num_units, out, lse,
 *   workspace, workspace_bytes, stream) on the same stream.
 * Errors: as for mla_plan_sizes / mla_get_metadata / mla_decode_fwd
 *   (MLA_ERR_UNSUPPORTED for topk > 2048, h_q not a multiple of 16).
 */
int mla_sparse_plan_sizes(int batch, int s_q, int h_q, int topk, int num_cus, int* num_units,
                          size_t* meta_bytes, size_t* splits_bytes, size_t* workspace_bytes);
int mla_get_metadata_sparse(const int32_t* topk_lens, int batch, int s_q, int h_q, int topk, int num_units,
                            int32_t* tile_meta, int32_t* num_splits, void* stream);
int mla_decode_sparse_fwd(const void* q, const void* kcache, int64_t nblocks,
                          const int32_t* block_table, int max_blocks,
                          const int32_t* indices, const int32_t* topk_lens, int topk,
                          int batch, int s_q, int h_q, float softmax_scale,
                          const int32_t* tile_meta, const int32_t* num_splits, int num_units,
                          void* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream);
int mla_decode_sparse_fwd_splits(const void* q, const void* kcache, int64_t nblocks,
                                 const int32_t* block_table, int max_blocks,
                                 const int32_t* indices, const int32_t* topk_lens, int topk,
                                 int batch, int s_q, int h_q, float softmax_scale,
                                 const int32_t* tile_meta, const int32_t* num_splits, int num_units,
                                 void* out, float* lse, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * FP8 latent cache: cached rows stored as 8-bit floats with one float32 scale
 * per row, half the bytes of the bf16 cache -- the FP8 support the FlashMLA
 * explainer (theflyingbirds.in) lists under section 9, "Future Directions",
 * to cut memory further. The pages fix no format; this library uses:
 *   codes: uint8 [nblocks, 64, 576], OCP E4M3 (sign, 4 exponent bits with
 *     bias 7, 3 mantissa bits, subnormals, no infinities, 0x7F/0xFF NaN);
 *   scales: float32 [nblocks, 64]; cached value = E4M3(code) * scale.
 * The attention is that of mla_decode_fwd over the decoded values (queries
 * stay bf16); rows no query may read may hold anything, NaN included.
 *
 * mla_fp8_plan_sizes / mla_get_metadata_fp8: the plan for this decode; the
 *   FP8 decode uses the geometry of the bf16 one (64 query rows per
 *   workgroup when s_q*h_q is a multiple of 64, else 16), so these return
 *   exactly what mla_plan_sizes / mla_get_metadata return.
 * mla_decode_fp8_fwd: as mla_decode_fwd with kcache replaced by (kcodes,
 *   kscale); both 16-byte aligned.
 * mla_decode_fp8_fwd_splits: its decode kernel alone (same arguments and
 *   checks); mla_decode_fp8_fwd is exactly it followed by mla_combine_splits
 *   with the same batch, s_q, h_q, plan and workspace on the same stream.
 * mla_append_kv_fp8: as mla_append_kv, but each new bf16 row is quantized
 *   into the FP8 cache: amax = its largest magnitude, scale = amax / 448 and
 *   code = E4M3 nearest (ties to even) to x * (448 / amax), the two quotients
 *   correctly rounded float32 and the product one float32 multiply; a row of
 *   zeros gets scale 0 and codes 0. Rows must be finite. kcodes 16-byte and
 *   kscale 4-byte aligned.
 * Errors: as for the bf16 calls.
 */
int mla_fp8_plan_sizes(int batch, int s_q, int h_q, int num_cus, int* num_units,
                       size_t* meta_bytes, size_t* splits_bytes, size_t* workspace_bytes);
int mla_get_metadata_fp8(const int32_t* cache_seqlens, int batch, int s_q, int h_q, int num_units,
                         int32_t* tile_meta, int32_t* num_splits, void* stream);
int mla_decode_fp8_fwd(const void* q, const void* kcodes, const float* kscale, int64_t nblocks,
                       const int32_t* block_table, int max_blocks,
                       const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                       float softmax_scale, int causal,
                       const int32_t* tile_meta, const int32_t* num_splits, int num_units,
                       void* out, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream);
int mla_decode_fp8_fwd_splits(const void* q, const void* kcodes, const float* kscale, int64_t nblocks,
                              const int32_t* block_table, int max_blocks,
                              const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                              float softmax_scale, int causal,
                              const int32_t* tile_meta, const int32_t* num_splits, int num_units,
                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream);
int mla_append_kv_fp8(void* kcodes, float* kscale, int64_t nblocks, const int32_t* block_table, int max_blocks,
                      const int32_t* cache_seqlens, const void* new_rows, int batch, int s_new, void* stream);

/*
 * Cache append: writes the new tokens' cached rows into their blocks, the
 * step that precedes decode attention over them (the cache grows by the new
 * tokens' entries each step: "OpenSourceWeek Day 1: FlashMLA", "How KV
 * Caching Works?"; blocks found through the block table: FlashMLA
 * explainer, section 4.3.2 "Paged KV Cache").
 *   kcache: device bf16 [nblocks, 64, 576], 16-byte aligned; written only at
 *     the new rows' positions.
 *   block_table: device int32 [batch, max_blocks].
 *   cache_seqlens: device int32 [batch], lengths INCLUDING the new tokens
 *     (the same array mla_decode_fwd then takes).
 *   new_rows: device bf16 [batch, s_new, 576], 16-byte aligned. Row i of
 *     sequence b goes to token position L_b - s_new + i (so the new tokens are
 *     the last s_new positions, as mla_decode_fwd reads them); rows whose
 *     position would be negative (L_b < s_new) are skipped.
 * One kernel on `stream`. Contract the host cannot check: block_table[b][j]
 * is a valid block for every block the new positions fall in, and no two
 * new rows map to the same cache row.
 * Errors: MLA_ERR_INVALID_ARG (null or misaligned pointer, non-positive
 *   size), MLA_ERR_UNSUPPORTED (more than 2^33 rows), MLA_ERR_HIP.
 */
int mla_append_kv(void* kcache, int64_t nblocks, const int32_t* block_table, int max_blocks,
                  const int32_t* cache_seqlens, const void* new_rows, int batch, int s_new, void* stream);

/*
 * Paged block pool: host-side bookkeeping of which physical cache blocks
 * belong to which sequence, so that a sequence's blocks need not be
 * contiguous and freed blocks are reused (FlashMLA explainer, section 4.3.2
 * "Paged KV Cache": fixed-size pages allocated on demand, like virtual
 * memory). The pool allocates host memory only and makes no HIP call; the
 * caller copies the tables it produces to the device. A pool is not
 * thread-safe: calls on one pool must not overlap.
 *
 * mla_block_pool_create: a pool of physical blocks [0, nblocks) for
 *   sequence slots [0, max_seqs), each of at most max_blocks_per_seq blocks.
 *   Blocks are handed out lowest id first; freed blocks are reused last
 *   freed first. *pool receives the handle (NULL on error).
 * mla_block_pool_reserve: make slot `seq` hold ceil(new_len / 64) blocks and
 *   set its length to new_len: blocks are appended when it grows and the
 *   tail blocks freed when it shrinks; kept blocks keep their ids, so rows
 *   already cached stay where they are. MLA_ERR_OUT_OF_BLOCKS if the free
 *   blocks do not suffice (the pool is left unchanged).
 * mla_block_pool_release: reserve(seq, 0): frees all blocks of the slot.
 * mla_block_pool_free_blocks: number of free blocks (-1 for NULL).
 * mla_block_pool_table: for slots seqs[0..n), writes row k of table (host
 *   int32 [n, max_blocks]) = the slot's block ids, padded with -1, and
 *   lens[k] = its length (lens may be NULL); MLA_ERR_INVALID_ARG if a slot
 *   holds more than max_blocks blocks.
 * Errors: MLA_ERR_INVALID_ARG (NULL pool, slot out of range, negative
 *   length, more than max_blocks_per_seq blocks), MLA_ERR_OUT_OF_MEMORY.
 */
int mla_block_pool_create(int64_t nblocks, int max_seqs, int max_blocks_per_seq, void** pool);
void mla_block_pool_destroy(void* pool);
int mla_block_pool_reserve(void* pool, int seq, int new_len);
int mla_block_pool_release(void* pool, int seq);
int64_t mla_block_pool_free_blocks(const void* pool);
int mla_block_pool_table(const void* pool, const int32_t* seqs, int n, int max_blocks, int32_t* table,
                         int32_t* lens);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PAGED_LATENT_H */
