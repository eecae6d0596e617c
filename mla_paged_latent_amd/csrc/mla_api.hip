// C ABI of the library: host-side argument checks, buffer sizing and kernel
// launches. Every check runs before anything is enqueued.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>
#include <vector>

#include "../../include/mla_paged_latent.h"
#include "mla_common.h"

namespace mla {
void plan_host(const int32_t* seqlens, int batch, int rows_wg, int num_units, int32_t* meta, int32_t* splits);
hipError_t launch_plan(const int32_t* seqlens, int batch, int rows_wg, int num_units, int32_t* meta,
                       int32_t* splits, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int num_units, int head_groups, int rows_wg, hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);
hipError_t launch_decode_sparse(const DecodeParams& p, int num_units, int head_groups, hipStream_t stream);
hipError_t launch_decode_fp8(const DecodeParams& p, int num_units, int head_groups, int rows_wg, hipStream_t stream);
}  // namespace mla

namespace {

constexpr int kMaxBatch = 16384;     // the device planner keeps two int arrays of batch+1 in LDS

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

int check_shape(int batch, int s_q, int h_q)
{
    if (batch < 1 || s_q < 1 || h_q < 1) return MLA_ERR_INVALID_ARG;
    if (batch > kMaxBatch) return MLA_ERR_UNSUPPORTED;
    const long rows = (long)s_q * h_q;
    if (rows % 16 != 0 || rows > mla::kMaxRows) return MLA_ERR_UNSUPPORTED;
    return MLA_OK;
}

struct Geometry {
    int rows_total, rows_wg, head_groups;
    bool by_sequence;
};

Geometry geometry(int s_q, int h_q)
{
    Geometry g;
    g.rows_total = s_q * h_q;
    g.rows_wg = mla::rows_per_wg(g.rows_total);
    g.head_groups = g.rows_total / g.rows_wg;
    g.by_sequence = mla::plan_by_sequence(g.rows_wg);
    return g;
}

// Per-sequence plans need at least one unit per sequence plus one to spread.
int check_units(const Geometry& geo, int batch, int num_units)
{
    if (num_units < 1) return MLA_ERR_INVALID_ARG;
    if (geo.by_sequence && num_units < batch + 1) return MLA_ERR_INVALID_ARG;
    return MLA_OK;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace: partial outputs for at most num_units + batch (unit, sequence)
// segments -- each unit boundary adds at most one segment to a sequence.
void workspace_layout(int batch, int rows_total, int num_units, size_t* part_o_bytes, size_t* total)
{
    const size_t slots = (size_t)num_units + (size_t)batch;
    *part_o_bytes = round_up(slots * rows_total * mla::kDv * sizeof(float), 256);
    *total = *part_o_bytes + round_up(slots * rows_total * sizeof(float), 256);
}

// The device-side contract of the decode calls on host arrays: 0 <= L_b <=
// 64 * max_blocks and block_table[b][j] in [0, nblocks) for j < ceil(L_b / 64).
int check_inputs(const int32_t* seqlens, int batch, const int32_t* table, int max_blocks, int64_t nblocks,
                 int* bad_seq)
{
    for (int b = 0; b < batch; ++b) {
        const int L = seqlens[b];
        bool ok = L >= 0 && (int64_t)L <= (int64_t)mla::kPage * max_blocks;
        for (int j = 0; ok && j < mla::blocks_of(L); ++j) {
            const int page = table[(size_t)b * max_blocks + j];
            ok = page >= 0 && page < nblocks;
        }
        if (!ok) {
            if (bad_seq) *bad_seq = b;
            return MLA_ERR_INVALID_ARG;
        }
    }
    if (bad_seq) *bad_seq = -1;
    return MLA_OK;
}

// With MLA_DEBUG_CHECK set (and not "0") in the environment, the decode calls
// copy cache_seqlens and block_table to the host and check the contract
// before anything is enqueued (a synchronising copy: for debugging only).
int debug_check_device_inputs(const int32_t* seqlens, int batch, const int32_t* table, int max_blocks,
                              int64_t nblocks, hipStream_t stream)
{
    const char* env = getenv("MLA_DEBUG_CHECK");
    if (!env || !env[0] || (env[0] == '0' && !env[1])) return MLA_OK;
    std::vector<int32_t> lens(batch), tab((size_t)batch * max_blocks);
    if (hipMemcpyAsync(lens.data(), seqlens, lens.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipMemcpyAsync(tab.data(), table, tab.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return MLA_ERR_HIP;
    return check_inputs(lens.data(), batch, tab.data(), max_blocks, nblocks, nullptr);
}

}  // namespace

extern "C" {

int mla_check_inputs_host(const int32_t* cache_seqlens, int batch, const int32_t* block_table, int max_blocks,
                          int64_t nblocks, int* bad_seq)
{
    if (!cache_seqlens || !block_table || batch < 1 || max_blocks < 1 || nblocks < 1) return MLA_ERR_INVALID_ARG;
    return check_inputs(cache_seqlens, batch, block_table, max_blocks, nblocks, bad_seq);
}

const char* mla_status_string(int status)
{
    switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, or non-positive size)";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape (s_q*h_q must be a multiple of 16 in [16, 1024], batch <= 16384)";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than mla_plan_sizes reports";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_OUT_OF_BLOCKS: return "block pool has too few free blocks";
    case MLA_ERR_OUT_OF_MEMORY: return "host allocation failed";
    default: return "unknown status";
    }
}

int mla_plan_sizes(int batch, int s_q, int h_q, int num_cus, int* num_units, size_t* meta_bytes,
                   size_t* splits_bytes, size_t* workspace_bytes)
{
    int rc = check_shape(batch, s_q, h_q);
    if (rc != MLA_OK) return rc;
    if (num_cus <= 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
        if (hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return MLA_ERR_HIP;
        if (num_cus <= 0) return MLA_ERR_HIP;
    }
    const Geometry geo = geometry(s_q, h_q);
    // one workgroup per CU (the block buffers fill most of the LDS); the 16-row
    // kernels' per-sequence plans take 7/8 of the CUs (fewer, longer units: fewer
    // split partials to write and merge, and the remaining CUs still saturate
    // HBM), and need at least one unit per sequence and one to spare
    const int cus = geo.by_sequence ? num_cus - num_cus / 8 : num_cus;
    int units = cus / geo.head_groups;
    if (units < 1) units = 1;
    if (geo.by_sequence && units < batch + 1) units = batch + 1;
    size_t part_o = 0, total = 0;
    workspace_layout(batch, geo.rows_total, units, &part_o, &total);
    if (num_units) *num_units = units;
    if (meta_bytes) *meta_bytes = (size_t)units * MLA_META_INTS * sizeof(int32_t);
    if (splits_bytes) *splits_bytes = (size_t)(batch + 1) * sizeof(int32_t);
    if (workspace_bytes) *workspace_bytes = total;
    return MLA_OK;
}

int mla_workspace_bytes(int batch, int s_q, int h_q, int num_units, size_t* workspace_bytes)
{
    int rc = check_shape(batch, s_q, h_q);
    if (rc != MLA_OK) return rc;
    if (!workspace_bytes || check_units(geometry(s_q, h_q), batch, num_units) != MLA_OK) return MLA_ERR_INVALID_ARG;
    size_t part_o = 0;
    workspace_layout(batch, s_q * h_q, num_units, &part_o, workspace_bytes);
    return MLA_OK;
}

int mla_get_metadata(const int32_t* cache_seqlens, int batch, int s_q, int h_q, int num_units,
                     int32_t* tile_meta, int32_t* num_splits, void* stream)
{
    int rc = check_shape(batch, s_q, h_q);
    if (rc != MLA_OK) return rc;
    if (!cache_seqlens || !tile_meta || !num_splits) return MLA_ERR_INVALID_ARG;
    const Geometry geo = geometry(s_q, h_q);
    if (check_units(geo, batch, num_units) != MLA_OK) return MLA_ERR_INVALID_ARG;
    if (mla::launch_plan(cache_seqlens, batch, geo.rows_wg, num_units, tile_meta, num_splits,
                         (hipStream_t)stream) != hipSuccess)
        return MLA_ERR_HIP;
    return MLA_OK;
}

int mla_get_metadata_host(const int32_t* cache_seqlens, int batch, int s_q, int h_q, int num_units,
                          int32_t* tile_meta, int32_t* num_splits)
{
    int rc = check_shape(batch, s_q, h_q);
    if (rc != MLA_OK) return rc;
    if (!cache_seqlens || !tile_meta || !num_splits) return MLA_ERR_INVALID_ARG;
    const Geometry geo = geometry(s_q, h_q);
    if (check_units(geo, batch, num_units) != MLA_OK) return MLA_ERR_INVALID_ARG;
    mla::plan_host(cache_seqlens, batch, geo.rows_wg, num_units, tile_meta, num_splits);
    return MLA_OK;
}

}  // extern "C"

namespace {

int setup_decode(const void* q, const void* kcache, int64_t nblocks, const int32_t* block_table, int max_blocks,
                 const int32_t* cache_seqlens, int batch, int s_q, int h_q, float softmax_scale, int causal,
                 const int32_t* tile_meta, const int32_t* num_splits, int num_units, void* out, float* lse,
                 void* workspace, size_t workspace_bytes, mla::DecodeParams* p, Geometry* geo_out)
{
    int rc = check_shape(batch, s_q, h_q);
    if (rc != MLA_OK) return rc;
    if (!q || !kcache || !block_table || !cache_seqlens || !tile_meta || !num_splits || !out || !lse ||
        !workspace)
        return MLA_ERR_INVALID_ARG;
    if (nblocks < 1 || max_blocks < 1 || !isfinite(softmax_scale)) return MLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kcache) || !aligned16(out) || !aligned16(workspace) || ((uintptr_t)lse & 3u))
        return MLA_ERR_INVALID_ARG;
    const Geometry geo = geometry(s_q, h_q);
    if (check_units(geo, batch, num_units) != MLA_OK) return MLA_ERR_INVALID_ARG;
    size_t part_o = 0, total = 0;
    workspace_layout(batch, geo.rows_total, num_units, &part_o, &total);
    if (workspace_bytes < total) return MLA_ERR_WORKSPACE_TOO_SMALL;

    p->q = (const uint16_t*)q;
    p->kcache = (const uint16_t*)kcache;
    p->block_table = block_table;
    p->seqlens = cache_seqlens;
    p->meta = tile_meta;
    p->splits = num_splits;
    p->out = (uint16_t*)out;
    p->lse = lse;
    p->part_o = (float*)workspace;
    p->part_lse = (float*)((char*)workspace + part_o);
    p->nblocks = nblocks;
    p->max_blocks = max_blocks;
    p->batch = batch;
    p->s_q = s_q;
    p->h_q = h_q;
    p->rows_total = geo.rows_total;
    p->causal = causal ? 1 : 0;
    p->scale_log2 = softmax_scale * 1.4426950408889634f;
    p->indices = nullptr;
    p->topk = 0;
    p->sq_real = 1;
    p->kscale = nullptr;
    *geo_out = geo;
    return MLA_OK;
}

int run_combine(const mla::DecodeParams& p, hipStream_t st)
{
    mla::CombineParams c;
    c.splits = p.splits;
    c.part_o = p.part_o;
    c.part_lse = p.part_lse;
    c.out = p.out;
    c.lse = p.lse;
    c.batch = p.batch;
    c.rows_total = p.rows_total;
    return mla::launch_combine(c, st) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

extern "C" {

int mla_decode_fwd(const void* q, const void* kcache, int64_t nblocks, const int32_t* block_table,
                   int max_blocks, const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                   float softmax_scale, int causal, const int32_t* tile_meta, const int32_t* num_splits,
                   int num_units, void* out, float* lse, void* workspace, size_t workspace_bytes,
                   void* stream)
{
    mla::DecodeParams p;
    Geometry geo;
    int rc = setup_decode(q, kcache, nblocks, block_table, max_blocks, cache_seqlens, batch, s_q, h_q,
                          softmax_scale, causal, tile_meta, num_splits, num_units, out, lse, workspace,
                          workspace_bytes, &p, &geo);
    if (rc != MLA_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    rc = debug_check_device_inputs(cache_seqlens, batch, block_table, max_blocks, nblocks, st);
    if (rc != MLA_OK) return rc;
    if (mla::launch_decode(p, num_units, geo.head_groups, geo.rows_wg, st) != hipSuccess) return MLA_ERR_HIP;
    return run_combine(p, st);
}

int mla_decode_fwd_splits(const void* q, const void* kcache, int64_t nblocks, const int32_t* block_table,
                          int max_blocks, const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                          float softmax_scale, int causal, const int32_t* tile_meta, const int32_t* num_splits,
                          int num_units, void* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream)
{
    mla::DecodeParams p;
    Geometry geo;
    int rc = setup_decode(q, kcache, nblocks, block_table, max_blocks, cache_seqlens, batch, s_q, h_q,
                          softmax_scale, causal, tile_meta, num_splits, num_units, out, lse, workspace,
                          workspace_bytes, &p, &geo);
    if (rc != MLA_OK) return rc;
    rc = debug_check_device_inputs(cache_seqlens, batch, block_table, max_blocks, nblocks, (hipStream_t)stream);
    if (rc != MLA_OK) return rc;
    if (mla::launch_decode(p, num_units, geo.head_groups, geo.rows_wg, (hipStream_t)stream) != hipSuccess)
        return MLA_ERR_HIP;
    return MLA_OK;
}

int mla_combine_splits(const int32_t* num_splits, int batch, int s_q, int h_q, int num_units, void* out,
                       float* lse, void* workspace, size_t workspace_bytes, void* stream)
{
    int rc = check_shape(batch, s_q, h_q);
    if (rc != MLA_OK) return rc;
    if (!num_splits || !out || !lse || !workspace) return MLA_ERR_INVALID_ARG;
    if (!aligned16(out) || !aligned16(workspace) || ((uintptr_t)lse & 3u)) return MLA_ERR_INVALID_ARG;
    const Geometry geo = geometry(s_q, h_q);
    if (check_units(geo, batch, num_units) != MLA_OK) return MLA_ERR_INVALID_ARG;
    size_t part_o = 0, total = 0;
    workspace_layout(batch, geo.rows_total, num_units, &part_o, &total);
    if (workspace_bytes < total) return MLA_ERR_WORKSPACE_TOO_SMALL;
    mla::DecodeParams p;
    p.splits = num_splits;
    p.part_o = (float*)workspace;
    p.part_lse = (float*)((char*)workspace + part_o);
    p.out = (uint16_t*)out;
    p.lse = lse;
    p.batch = batch;
    p.rows_total = geo.rows_total;
    return run_combine(p, (hipStream_t)stream);
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free decode
//
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops): the split partials live in one file-scope device
// array instead of a caller workspace. Each GPU the library runs on holds its
// own copy of the array until the process ends; host code reaches it only
// through the address hipGetSymbolAddress returns on that device (the name
// itself is a host-side stand-in). Every call on a GPU shares that GPU's
// array, so calls that overlap in time on one GPU race.

static __device__ __attribute__((aligned(256))) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and kept.
int scratch_of_current_device(void** ptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return MLA_ERR_HIP;
        g_scratch[dev] = addr;
    }
    *ptr = g_scratch[dev];
    return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_fwd_noalloc(const void* q, const void* kcache, int64_t nblocks, const int32_t* block_table,
                           int max_blocks, const int32_t* cache_seqlens, int batch, int s_q, int h_q,
                           float softmax_scale, int causal, const int32_t* tile_meta, const int32_t* num_splits,
                           int num_units, void* out, float* lse, void* stream)
{
    // every argument and the size this call needs are checked before any HIP
    // call; a 256-aligned stand-in takes the workspace's place in the checks
    mla::DecodeParams p;
    Geometry geo;
    int rc = setup_decode(q, kcache, nblocks, block_table, max_blocks, cache_seqlens, batch, s_q, h_q,
                          softmax_scale, causal, tile_meta, num_splits, num_units, out, lse, (void*)(uintptr_t)256,
                          MLA_NOALLOC_SCRATCH_BYTES, &p, &geo);
    if (rc != MLA_OK) return rc;
    void* ws = nullptr;
    rc = scratch_of_current_device(&ws);
    if (rc != MLA_OK) return rc;
    size_t part_o = 0, total = 0;
    workspace_layout(batch, geo.rows_total, num_units, &part_o, &total);
    p.part_o = (float*)ws;
    p.part_lse = (float*)((char*)ws + part_o);
    hipStream_t st = (hipStream_t)stream;
    if (mla::launch_decode(p, num_units, geo.head_groups, geo.rows_wg, st) != hipSuccess) return MLA_ERR_HIP;
    return run_combine(p, st);
}

}  // extern "C"

// ---------------------------------------------------------------- sparse decode
//
// A sparse batch of `batch` sequences with s_q new tokens each is planned and
// decoded as a batch of batch*s_q token lists of h_q rows each (the streaming
// kernel with its per-list plan); the lists' lengths play the part of
// cache_seqlens.

namespace {

constexpr int kMaxTopk = 2048;

int check_sparse_shape(int batch, int s_q, int h_q, int topk)
{
    if (batch < 1 || s_q < 1 || h_q < 1 || topk < 1) return MLA_ERR_INVALID_ARG;
    if ((long)batch * s_q > kMaxBatch || h_q % 16 != 0 || h_q > mla::kMaxRows || topk > kMaxTopk)
        return MLA_ERR_UNSUPPORTED;
    return MLA_OK;
}

}  // namespace

extern "C" {

int mla_sparse_plan_sizes(int batch, int s_q, int h_q, int topk, int num_cus, int* num_units, size_t* meta_bytes,
                          size_t* splits_bytes, size_t* workspace_bytes)
{
    int rc = check_sparse_shape(batch, s_q, h_q, topk);
    if (rc != MLA_OK) return rc;
    if (num_cus <= 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
        if (hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return MLA_ERR_HIP;
        if (num_cus <= 0) return MLA_ERR_HIP;
    }
    const int lists = batch * s_q;
    int units = num_cus / (h_q / 16);
    if (units < lists + 1) units = lists + 1;
    size_t part_o = 0, total = 0;
    workspace_layout(lists, h_q, units, &part_o, &total);
    if (num_units) *num_units = units;
    if (meta_bytes) *meta_bytes = (size_t)units * mla::kMetaInts * sizeof(int32_t);
    if (splits_bytes) *splits_bytes = (size_t)(lists + 1) * sizeof(int32_t);
    if (workspace_bytes) *workspace_bytes = total;
    return MLA_OK;
}

int mla_get_metadata_sparse(const int32_t* topk_lens, int batch, int s_q, int h_q, int topk, int num_units,
                            int32_t* tile_meta, int32_t* num_splits, void* stream)
{
    int rc = check_sparse_shape(batch, s_q, h_q, topk);
    if (rc != MLA_OK) return rc;
    if (!topk_lens || !tile_meta || !num_splits) return MLA_ERR_INVALID_ARG;
    if (num_units < batch * s_q + 1) return MLA_ERR_INVALID_ARG;
    if (mla::launch_plan(topk_lens, batch * s_q, 16, num_units, tile_meta, num_splits, (hipStream_t)stream) !=
        hipSuccess)
        return MLA_ERR_HIP;
    return MLA_OK;
}

}  // extern "C"

namespace {

// The sparse decode kernel, then (with `combine`) the split combine.
int decode_sparse(const void* q, const void* kcache, int64_t nblocks, const int32_t* block_table, int max_blocks,
                  const int32_t* indices, const int32_t* topk_lens, int topk, int batch, int s_q, int h_q,
                  float softmax_scale, const int32_t* tile_meta, const int32_t* num_splits, int num_units, void* out,
                  float* lse, void* workspace, size_t workspace_bytes, void* stream, bool combine)
{
    int rc = check_sparse_shape(batch, s_q, h_q, topk);
    if (rc != MLA_OK) return rc;
    if (!q || !kcache || !block_table || !indices || !topk_lens || !tile_meta || !num_splits || !out || !lse ||
        !workspace)
        return MLA_ERR_INVALID_ARG;
    if (nblocks < 1 || nblocks > 0x7fffffff / mla::kPage || max_blocks < 1 || !isfinite(softmax_scale))
        return MLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kcache) || !aligned16(out) || !aligned16(workspace) || ((uintptr_t)lse & 3u))
        return MLA_ERR_INVALID_ARG;
    const int lists = batch * s_q;
    if (num_units < lists + 1) return MLA_ERR_INVALID_ARG;
    size_t part_o = 0, total = 0;
    workspace_layout(lists, h_q, num_units, &part_o, &total);
    if (workspace_bytes < total) return MLA_ERR_WORKSPACE_TOO_SMALL;
    mla::DecodeParams p;
    p.q = (const uint16_t*)q;
    p.kcache = (const uint16_t*)kcache;
    p.block_table = block_table;
    p.seqlens = topk_lens;
    p.meta = tile_meta;
    p.splits = num_splits;
    p.out = (uint16_t*)out;
    p.lse = lse;
    p.part_o = (float*)workspace;
    p.part_lse = (float*)((char*)workspace + part_o);
    p.nblocks = nblocks;
    p.max_blocks = max_blocks;
    p.batch = lists;
    p.s_q = 1;
    p.h_q = h_q;
    p.rows_total = h_q;
    p.causal = 0;
    p.scale_log2 = softmax_scale * 1.4426950408889634f;
    p.indices = indices;
    p.topk = topk;
    p.sq_real = s_q;
    p.kscale = nullptr;
    hipStream_t st = (hipStream_t)stream;
    if (mla::launch_decode_sparse(p, num_units, h_q / 16, st) != hipSuccess) return MLA_ERR_HIP;
    return combine ? run_combine(p, st) : MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_sparse_fwd(const void* q, const void* kcache, int64_t nblocks, const int32_t* block_table,
                          int max_blocks, const int32_t* indices, const int32_t* topk_lens, int topk, int batch,
                          int s_q, int h_q, float softmax_scale, const int32_t* tile_meta,
                          const int32_t* num_splits, int num_units, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream)
{
    return decode_sparse(q, kcache, nblocks, block_table, max_blocks, indices, topk_lens, topk, batch, s_q, h_q,
                         softmax_scale, tile_meta, num_splits, num_units, out, lse, workspace, workspace_bytes, stream,
                         true);
}

int mla_decode_sparse_fwd_splits(const void* q, const void* kcache, int64_t nblocks, const int32_t* block_table,
                                 int max_blocks, const int32_t* indices, const int32_t* topk_lens, int topk,
                                 int batch, int s_q, int h_q, float softmax_scale, const int32_t* tile_meta,
                                 const int32_t* num_splits, int num_units, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream)
{
    return decode_sparse(q, kcache, nblocks, block_table, max_blocks, indices, topk_lens, topk, batch, s_q, h_q,
                         softmax_scale, tile_meta, num_splits, num_units, out, lse, workspace, workspace_bytes, stream,
                         false);
}

}  // extern "C"

// ---------------------------------------------------------------- FP8 cache decode
//
// The FP8 cache is decoded with the same geometry and plan as the bf16 cache:
// 64-row workgroups (the FP8 wide kernel) when s_q * h_q is a multiple of 64,
// else 16-row workgroups (the FP8 streaming kernel).

extern "C" {

int mla_fp8_plan_sizes(int batch, int s_q, int h_q, int num_cus, int* num_units, size_t* meta_bytes,
                       size_t* splits_bytes, size_t* workspace_bytes)
{
    return mla_plan_sizes(batch, s_q, h_q, num_cus, num_units, meta_bytes, splits_bytes, workspace_bytes);
}

int mla_get_metadata_fp8(const int32_t* cache_seqlens, int batch, int s_q, int h_q, int num_units,
                         int32_t* tile_meta, int32_t* num_splits, void* stream)
{
    return mla_get_metadata(cache_seqlens, batch, s_q, h_q, num_units, tile_meta, num_splits, stream);
}

}  // extern "C"

namespace {

// The FP8 decode kernel, then (with `combine`) the split combine.
int decode_fp8(const void* q, const void* kcodes, const float* kscale, int64_t nblocks, const int32_t* block_table,
               int max_blocks, const int32_t* cache_seqlens, int batch, int s_q, int h_q, float softmax_scale,
               int causal, const int32_t* tile_meta, const int32_t* num_splits, int num_units, void* out, float* lse,
               void* workspace, size_t workspace_bytes, void* stream, bool combine)
{
    int rc = check_shape(batch, s_q, h_q);
    if (rc != MLA_OK) return rc;
    if (!q || !kcodes || !kscale || !block_table || !cache_seqlens || !tile_meta || !num_splits || !out || !lse ||
        !workspace)
        return MLA_ERR_INVALID_ARG;
    if (nblocks < 1 || max_blocks < 1 || !isfinite(softmax_scale)) return MLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kcodes) || !aligned16(kscale) || !aligned16(out) || !aligned16(workspace) ||
        ((uintptr_t)lse & 3u))
        return MLA_ERR_INVALID_ARG;
    const Geometry geo = geometry(s_q, h_q);
    if (check_units(geo, batch, num_units) != MLA_OK) return MLA_ERR_INVALID_ARG;
    const int rows = s_q * h_q;
    size_t part_o = 0, total = 0;
    workspace_layout(batch, rows, num_units, &part_o, &total);
    if (workspace_bytes < total) return MLA_ERR_WORKSPACE_TOO_SMALL;
    mla::DecodeParams p;
    p.q = (const uint16_t*)q;
    p.kcache = (const uint16_t*)kcodes;
    p.block_table = block_table;
    p.seqlens = cache_seqlens;
    p.meta = tile_meta;
    p.splits = num_splits;
    p.out = (uint16_t*)out;
    p.lse = lse;
    p.part_o = (float*)workspace;
    p.part_lse = (float*)((char*)workspace + part_o);
    p.nblocks = nblocks;
    p.max_blocks = max_blocks;
    p.batch = batch;
    p.s_q = s_q;
    p.h_q = h_q;
    p.rows_total = rows;
    p.causal = causal ? 1 : 0;
    p.scale_log2 = softmax_scale * 1.4426950408889634f;
    p.indices = nullptr;
    p.topk = 0;
    p.sq_real = 1;
    p.kscale = kscale;
    hipStream_t st = (hipStream_t)stream;
    rc = debug_check_device_inputs(cache_seqlens, batch, block_table, max_blocks, nblocks, st);
    if (rc != MLA_OK) return rc;
    if (mla::launch_decode_fp8(p, num_units, geo.head_groups, geo.rows_wg, st) != hipSuccess) return MLA_ERR_HIP;
    return combine ? run_combine(p, st) : MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_fp8_fwd(const void* q, const void* kcodes, const float* kscale, int64_t nblocks,
                       const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens, int batch, int s_q,
                       int h_q, float softmax_scale, int causal, const int32_t* tile_meta, const int32_t* num_splits,
                       int num_units, void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream)
{
    return decode_fp8(q, kcodes, kscale, nblocks, block_table, max_blocks, cache_seqlens, batch, s_q, h_q,
                      softmax_scale, causal, tile_meta, num_splits, num_units, out, lse, workspace, workspace_bytes,
                      stream, true);
}

int mla_decode_fp8_fwd_splits(const void* q, const void* kcodes, const float* kscale, int64_t nblocks,
                              const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens, int batch,
                              int s_q, int h_q, float softmax_scale, int causal, const int32_t* tile_meta,
                              const int32_t* num_splits, int num_units, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream)
{
    return decode_fp8(q, kcodes, kscale, nblocks, block_table, max_blocks, cache_seqlens, batch, s_q, h_q,
                      softmax_scale, causal, tile_meta, num_splits, num_units, out, lse, workspace, workspace_bytes,
                      stream, false);
}

}  // extern "C"
