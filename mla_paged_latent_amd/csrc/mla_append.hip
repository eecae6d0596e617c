// Cache append and the paged block pool.
//
// Each decode step adds the new tokens' latent rows to the cache before they
// are attended over ("OpenSourceWeek Day 1: FlashMLA", bibleofai.com, "How
// KV Caching Works?"); the cache is paged in fixed 64-token blocks found
// through a per-sequence block table, allocated as a sequence grows and
// returned when it ends (FlashMLA explainer, theflyingbirds.in, section
// 4.3.2 "Paged KV Cache", the virtual-memory analogy).
//
//  * append_kernel: one wave per new row; the row's 1152 bytes are 72 chunks
//    of 16 B, lanes 0-63 take chunks 0-63 and lanes 0-7 also 64-71, so the
//    reads and the writes are whole 1 KB + 128 B runs. The new row is loaded
//    before (and beside) the sequence length and the block-table entry that
//    place it, which are wave-uniform scalar loads: two memory round trips per
//    row instead of three.
//  * BlockPool: host bookkeeping only (no HIP call): a LIFO free list of
//    physical block ids and, per sequence, its length and blocks in order.
#include <stdint.h>
#include <stdlib.h>

#include <new>
#include <vector>

#include "../../include/mla_paged_latent.h"
#include "mla_device.h"

namespace mla {
namespace {

// Max over the lane's 16-lane row with DPP (quad swaps, then the 8- and 16-lane
// mirrors), all in registers.
__device__ __forceinline__ float row16_max(float x)
{
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true)));   // quad [1,0,3,2]
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true)));   // quad [2,3,0,1]
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true)));  // row half mirror
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true)));  // row mirror
    return x;
}

typedef unsigned u32x4a __attribute__((ext_vector_type(4)));
typedef unsigned u32x2a __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256) void append_kernel(uint16_t* __restrict__ kcache, int64_t nblocks,
                                                     const int32_t* __restrict__ block_table, int max_blocks,
                                                     const int32_t* __restrict__ seqlens,
                                                     const uint16_t* __restrict__ rows, int batch, int s_new)
{
    const int lane = threadIdx.x & 63;
    const long r = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // new row b * s_new + i
    if (r >= (long)batch * s_new) return;
    // the row first (it needs nothing else); lanes 8-63 re-read chunks 64-71 of the
    // row, so the load is unconditional and nothing waits on it before the stores
    const u32x4a* src = (const u32x4a*)(rows + (size_t)r * kDqk);
    const u32x4a a = src[lane];
    const u32x4a c = src[64 + (lane & 7)];
    const int b = (int)(r / s_new);
    const int i = (int)(r - (long)b * s_new);
    const int pos = cload(seqlens + b) - s_new + i;              // its token position
    // rows of a sequence shorter than s_new, past the table or in a block outside
    // the cache are not written (the table is read at a valid index regardless)
    const bool in_table = pos >= 0 && (pos >> 6) < max_blocks;
    const int page = cload(block_table + (size_t)b * max_blocks + (in_table ? (pos >> 6) : 0));
    if (!in_table || page < 0 || page >= nblocks) return;
    u32x4a* dst = (u32x4a*)(kcache + ((size_t)page * kPage + (pos & (kPage - 1))) * kDqk);
    dst[lane] = a;
    if (lane < 8) dst[64 + lane] = c;
}

// FP8 append: one wave per new row. Lanes 0-63 hold bf16 columns 8l..8l+7 and
// lanes 0-7 also 512+8l..; the row's largest magnitude comes from a wave max;
// scale = amax / 448 and codes = E4M3(x * (448 / amax)), both quotients
// correctly rounded float32 and the product one float32 multiply, converted
// to E4M3 by the hardware (round to nearest even; |x * 448 / amax| <= 448 so
// nothing saturates). A zero row gets scale 0 and codes 0. The wave max is
// taken in registers (DPP within 16-lane rows, then lane swaps across rows).
__global__ __launch_bounds__(256) void append_fp8_kernel(unsigned char* __restrict__ codes, float* __restrict__ scales,
                                                         int64_t nblocks,
                                                         const int32_t* __restrict__ block_table, int max_blocks,
                                                         const int32_t* __restrict__ seqlens,
                                                         const uint16_t* __restrict__ rows, int batch, int s_new)
{
    const int lane = threadIdx.x & 63;
    const long r = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (r >= (long)batch * s_new) return;
    const u32x4a* src = (const u32x4a*)(rows + (size_t)r * kDqk);
    const u32x4a a = src[lane];                                  // the row first, as in append_kernel
    const u32x4a c8 = src[64 + (lane & 7)];
    const u32x4a c = lane < 8 ? c8 : u32x4a{0u, 0u, 0u, 0u};
    const int b = (int)(r / s_new);
    const int i = (int)(r - (long)b * s_new);
    const int pos = cload(seqlens + b) - s_new + i;
    const bool in_table = pos >= 0 && (pos >> 6) < max_blocks;
    const int page = cload(block_table + (size_t)b * max_blocks + (in_table ? (pos >> 6) : 0));
    if (!in_table || page < 0 || page >= nblocks) return;
    const size_t drow = (size_t)page * kPage + (pos & (kPage - 1));
    float x[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(a[k] << 16);
        x[2 * k + 1] = __uint_as_float(a[k] & 0xFFFF0000u);
        x[8 + 2 * k] = __uint_as_float(c[k] << 16);
        x[8 + 2 * k + 1] = __uint_as_float(c[k] & 0xFFFF0000u);
    }
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) m = fmaxf(m, fabsf(x[k]));
    m = xor32_max(xor16_max(row16_max(m)));                      // the row's largest magnitude, in every lane
    const float inv = m > 0.f ? __fdiv_rn(448.f, m) : 0.f;
    unsigned w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * k] * inv, x[4 * k + 1] * inv, 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * k + 2] * inv, x[4 * k + 3] * inv, v, true);
        w[k] = (unsigned)v;
    }
    unsigned* dst = (unsigned*)(codes + drow * kDqk);
    *(u32x2a*)(dst + 2 * lane) = u32x2a{w[0], w[1]};
    if (lane < 8) *(u32x2a*)(dst + 128 + 2 * lane) = u32x2a{w[2], w[3]};
    if (lane == 0) scales[drow] = m > 0.f ? __fdiv_rn(m, 448.f) : 0.f;
}

struct BlockPool {
    int64_t nblocks;
    int max_seqs;
    int max_blocks_per_seq;
    std::vector<int32_t> free_ids;                  // stack: the last entry is handed out next
    std::vector<std::vector<int32_t>> blocks;       // per sequence, in token order
    std::vector<int32_t> lens;
};

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

}  // namespace
}  // namespace mla

extern "C" {

int mla_append_kv(void* kcache, int64_t nblocks, const int32_t* block_table, int max_blocks,
                  const int32_t* cache_seqlens, const void* new_rows, int batch, int s_new, void* stream)
{
    if (!kcache || !block_table || !cache_seqlens || !new_rows) return MLA_ERR_INVALID_ARG;
    if (nblocks < 1 || max_blocks < 1 || batch < 1 || s_new < 1) return MLA_ERR_INVALID_ARG;
    if (!mla::aligned16(kcache) || !mla::aligned16(new_rows)) return MLA_ERR_INVALID_ARG;
    const long rows = (long)batch * s_new;
    if (rows > (long)0x7fffffff * 4 - 4) return MLA_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)((rows + 3) / 4));
    hipLaunchKernelGGL(mla::append_kernel, grid, dim3(256), 0, (hipStream_t)stream, (uint16_t*)kcache, nblocks,
                       block_table, max_blocks, cache_seqlens, (const uint16_t*)new_rows, batch, s_new);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_append_kv_fp8(void* codes, float* scales, int64_t nblocks, const int32_t* block_table, int max_blocks,
                      const int32_t* cache_seqlens, const void* new_rows, int batch, int s_new, void* stream)
{
    if (!codes || !scales || !block_table || !cache_seqlens || !new_rows) return MLA_ERR_INVALID_ARG;
    if (nblocks < 1 || max_blocks < 1 || batch < 1 || s_new < 1) return MLA_ERR_INVALID_ARG;
    if (!mla::aligned16(codes) || !mla::aligned16(new_rows) || ((uintptr_t)scales & 3u)) return MLA_ERR_INVALID_ARG;
    const long rows = (long)batch * s_new;
    if (rows > (long)0x7fffffff * 4 - 4) return MLA_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)((rows + 3) / 4));
    hipLaunchKernelGGL(mla::append_fp8_kernel, grid, dim3(256), 0, (hipStream_t)stream, (unsigned char*)codes,
                       scales, nblocks, block_table, max_blocks, cache_seqlens, (const uint16_t*)new_rows, batch,
                       s_new);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_block_pool_create(int64_t nblocks, int max_seqs, int max_blocks_per_seq, void** pool)
{
    if (!pool) return MLA_ERR_INVALID_ARG;
    *pool = nullptr;
    if (nblocks < 1 || nblocks > 0x7fffffff || max_seqs < 1 || max_blocks_per_seq < 1) return MLA_ERR_INVALID_ARG;
    mla::BlockPool* p = new (std::nothrow) mla::BlockPool;
    if (!p) return MLA_ERR_OUT_OF_MEMORY;
    try {
        p->nblocks = nblocks;
        p->max_seqs = max_seqs;
        p->max_blocks_per_seq = max_blocks_per_seq;
        p->free_ids.resize((size_t)nblocks);
        for (int64_t k = 0; k < nblocks; ++k) p->free_ids[(size_t)k] = (int32_t)(nblocks - 1 - k);
        p->blocks.resize((size_t)max_seqs);
        p->lens.assign((size_t)max_seqs, 0);
    } catch (...) {
        delete p;
        return MLA_ERR_OUT_OF_MEMORY;
    }
    *pool = p;
    return MLA_OK;
}

void mla_block_pool_destroy(void* pool) { delete (mla::BlockPool*)pool; }

int mla_block_pool_reserve(void* pool, int seq, int new_len)
{
    mla::BlockPool* p = (mla::BlockPool*)pool;
    if (!p || seq < 0 || seq >= p->max_seqs || new_len < 0) return MLA_ERR_INVALID_ARG;
    const long need = ((long)new_len + mla::kPage - 1) / mla::kPage;
    if (need > p->max_blocks_per_seq) return MLA_ERR_INVALID_ARG;
    std::vector<int32_t>& own = p->blocks[(size_t)seq];
    const long have = (long)own.size();
    if (need > have) {
        if ((long)p->free_ids.size() < need - have) return MLA_ERR_OUT_OF_BLOCKS;
        try {
            own.reserve((size_t)need);
        } catch (...) {
            return MLA_ERR_OUT_OF_MEMORY;
        }
        for (long k = have; k < need; ++k) {
            own.push_back(p->free_ids.back());
            p->free_ids.pop_back();
        }
    } else {
        for (long k = have; k > need; --k) {        // shrink: the tail blocks go back, last first
            p->free_ids.push_back(own.back());
            own.pop_back();
        }
    }
    p->lens[(size_t)seq] = new_len;
    return MLA_OK;
}

int mla_block_pool_release(void* pool, int seq) { return mla_block_pool_reserve(pool, seq, 0); }

int64_t mla_block_pool_free_blocks(const void* pool)
{
    const mla::BlockPool* p = (const mla::BlockPool*)pool;
    return p ? (int64_t)p->free_ids.size() : -1;
}

int mla_block_pool_table(const void* pool, const int32_t* seqs, int n, int max_blocks, int32_t* table,
                         int32_t* lens)
{
    const mla::BlockPool* p = (const mla::BlockPool*)pool;
    if (!p || !seqs || n < 1 || max_blocks < 1 || !table) return MLA_ERR_INVALID_ARG;
    for (int k = 0; k < n; ++k)
        if (seqs[k] < 0 || seqs[k] >= p->max_seqs || (long)p->blocks[(size_t)seqs[k]].size() > max_blocks)
            return MLA_ERR_INVALID_ARG;
    for (int k = 0; k < n; ++k) {
        const std::vector<int32_t>& own = p->blocks[(size_t)seqs[k]];
        int32_t* row = table + (size_t)k * max_blocks;
        for (int j = 0; j < max_blocks; ++j) row[j] = j < (int)own.size() ? own[(size_t)j] : -1;
        if (lens) lens[k] = p->lens[(size_t)seqs[k]];
    }
    return MLA_OK;
}

}  // extern "C"
