// MLA decode kernels for gfx950 (CDNA4): paged latent cache -> LDS -> bf16 MFMA.
//
// The method: decode-time attention of new queries over cached rows
// ("OpenSourceWeek Day 1: FlashMLA", bibleofai.com, "How KV Caching Works?")
// with one latent row per token shared by all heads (same page, "How MLA
// Optimizes Memory Usage?"), scaled dot-product softmax (FlashMLA explainer,
// theflyingbirds.in, section 4.1.1), 64-token pages behind a block table
// (explainer 4.3.2; bibleofai "Key Highlights"), blocks staged on chip and
// read with contiguous accesses (explainer 4.2.1-4.2.2), softmax fused with
// the two matrix products (explainer 4.2.3).
//
// Two decode kernels share the data path below; they differ in how the four
// waves of a workgroup divide the work.
//
//  * Streaming kernel (16 query rows per workgroup): every wave holds
//    all the workgroup's rows and streams its own 16-token sub-tiles through a
//    private two-slot LDS ring (direct global->LDS loads, no workgroup barrier
//    in the loop), so each CU keeps up to 8 x 18 KB of cache in flight. The
//    four waves' partial softmax states are merged once at the end. QK^T on
//    v_mfma_f32_16x16x32_bf16, PV on v_mfma_f32_16x16x16_bf16.
//  * Wide kernel (64 query rows, mla_decode_wide.hip): the workgroup's waves
//    share two 64-token block buffers in LDS (the block being computed and the
//    next one in flight); QK^T and PV on v_mfma_f32_32x32x16_bf16. A unit may
//    cover several sequences.
//
// Data path common to both:
//  * a cache block is 64 contiguous rows of 1152 B; in the streaming kernel an
//    LDS row is 72 chunks of 16 B plus one pad chunk (stride 1168 B), in the
//    wide kernel it is unpadded with chunk c of row r stored at c ^ f(r),
//    f(r) = ((r << 1) ^ (r >> 2)) mod 16 (chunks 64-71 by f's low three bits);
//  * S^T = K Q^T: K rows are the MFMA A operand (ds_read_b128), Q^T the B
//    operand held in VGPRs. The S^T accumulator layout (lane = query row,
//    4 tokens per element group) is exactly the P^T B operand of O^T = V^T P^T,
//    so P never leaves registers;
//  * V^T comes from ds_read_b64_tr_b16: within each 16-lane group, output lane
//    j element e is element j%4 of what source lane 4e + j/4 read, so source
//    lanes read 4 dims of 4 token rows and every output lane ends with one dim
//    of 4 tokens -- the MFMA A operand;
//  * the MFMA row <-> token map is permuted so that fragment reads and
//    transpose reads fall in distinct LDS bank groups: rows 0-7 of the 16-row
//    tiles are the even tokens and rows 8-15 the odd ones (stream_token); the
//    32-row tiles of the wide kernel use token(a) = 8(a/8) + 2(a%4) + (a/4)%2
//    with a chunk permutation of their own;
//  * scores are scaled into the exp2 domain; the running max is raised (and O
//    rescaled) only when a score exceeds it by more than 2^8, so P <= 256;
//  * rows past the end of a sequence are loaded from the block's first valid
//    row instead (finite data, masked to p = 0), so no LDS row holds garbage;
//  * scalars (plan rows, sequence lengths, split counts) are read with scalar
//    loads, and block-table entries 64 at a time with one vector load into a
//    register (readlane picks an entry), awaited before the copy pipeline starts
//    or together with a block copy that is awaited anyway, so that no wait in
//    the pipeline is for anything but block copies.
#include "mla_device.h"

namespace mla {

hipError_t launch_wide(const DecodeParams& p, dim3 grid, hipStream_t stream);       // mla_decode_wide.hip
hipError_t launch_wide_fp8(const DecodeParams& p, dim3 grid, hipStream_t stream);   // mla_decode_wide_fp8.hip

constexpr int kLdsRow = 1168;            // LDS row stride: 72 data chunks + 1 pad chunk of 16 B
constexpr int kRowSlots = 73;

// Token (0..15) of row a of the 16-row MFMA tiles of the streaming kernel:
// rows 0-7 are the even tokens, rows 8-15 the odd ones. The LDS serves a
// read from 16 groups of four banks and slot row t starts in group 9t mod 16
// (1168 = 73 x 16 B): a K fragment read (16 rows, one chunk) hits 16 groups for
// any order, and the first (second) 32 lanes of a V^T transpose read (8 rows,
// two adjacent chunks) hit 16 groups because their rows are the even (odd)
// tokens, whose groups 9t mod 16 are all even (odd).
__device__ __forceinline__ int stream_token(int a) { return 2 * (a & 7) + (a >> 3); }

// Copy the 16 rows of a run starting at gbase (wave-uniform; the first `valid`
// rows real) into an LDS slot of 1168-byte rows: copy i (first, first + step,
// ... < ninstr) fills slot chunks [64 i, 64 i + 64), chunk position q holding
// chunk q mod 73 of row q / 73; the pad chunk and rows >= valid repeat a real
// chunk. Every copy is issued from the scalar base plus a 32-bit lane offset,
// and q / 73 = (q * 898) >> 16 holds exactly for every q < 3649 (slots have
// 1216 positions), so the per-copy address work is a few full-rate 24-bit ops.
__device__ __forceinline__ void copy_rows(const unsigned char* gbase, int valid, unsigned slot, int first,
                                          int step, int ninstr, int lane)
{
    for (int i = first; i < ninstr; i += step) {
        const int q = i * 64 + lane;
        int r = (int)(__umul24((unsigned)q, 898u) >> 16);
        int c = q - kRowSlots * r;
        r = r < valid ? r : 0;
        c = c < kChunks ? c : 0;
        dma16s(gbase, (unsigned)(r * kRowBytes + c * 16), slot + (unsigned)i * 1024u);
    }
}

constexpr int kSlotA = 19 * 1024;        // 16 rows x 1168 B, rounded up to whole 1 KB copies
constexpr int kDmaA = 19;
constexpr int kLdsA = 8 * kSlotA;        // two slots per wave: 155,648 B

// Merge the four waves' (m, l, O) of a 16-row streaming workgroup and write
// the result. As soon as a wave is done with its slots it posts its 32 tiles
// (unscaled fp32, 32 KB) and its running max/sum per row into its own slot
// area; one workgroup barrier later wave w folds the four waves' tiles nt in
// [8w, 8w + 8) (dims [128w, 128w + 128)) and writes them. Register indices are
// static and only LDS and global addresses depend on the wave, so the code is
// executed by every wave alike (it runs once per launch, from a cold
// instruction cache). acc[nt] element i is dim 16 nt + 4 (lane / 16) + i of
// row lane % 16 of the workgroup's rows.
constexpr unsigned kPostML = 32768;      // a wave's posting: 32 fp32 tiles, then row max and row sum

__device__ __forceinline__ void stream_merge_store(const DecodeParams& p, const f32x4* acc, float mrun, float lrun,
                                                   unsigned lds0, unsigned slot0, int wave, int lane, int b, int slot,
                                                   int nsplit)
{
    constexpr int R = 16;
    const int g = lane >> 4;
    const int c16 = lane & 15;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");       // this wave's slot reads are done
    if (g == 0) {
        *(lds_f32*)(uintptr_t)(slot0 + kPostML + 4u * c16) = mrun;
        *(lds_f32*)(uintptr_t)(slot0 + kPostML + 64u + 4u * c16) = lrun;
    }
#pragma unroll
    for (int nt = 0; nt < 32; ++nt)
        *(lds_f32x4*)(uintptr_t)(slot0 + (unsigned)((nt * 64 + lane) * 16)) = acc[nt];
    wg_barrier();
    float mw[4], mall = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        mw[w] = *(const lds_f32*)(uintptr_t)(lds0 + (unsigned)(2 * w) * kSlotA + kPostML + 4u * c16);
        mall = fmaxf(mall, mw[w]);
    }
    float fw[4], lt = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        fw[w] = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - mall);
        lt += *(const lds_f32*)(uintptr_t)(lds0 + (unsigned)(2 * w) * kSlotA + kPostML + 64u + 4u * c16) * fw[w];
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float sw[4];                                            // weight of wave w's posting, 1/l folded in
#pragma unroll
    for (int w = 0; w < 4; ++w) sw[w] = fw[w] * inv;
    const int grow = blockIdx.y * R + c16;
    const unsigned tile0 = (unsigned)((8 * wave * 64 + lane) * 16);    // this wave's first tile in a posting
    f32x4 v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        v[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 4; ++w)
            v[t] += *(const lds_f32x4*)(uintptr_t)(lds0 + (unsigned)(2 * w) * kSlotA + tile0 + 1024u * t) * sw[w];
    }
    // tile 8 wave + t holds dims 128 wave + 16 t + 4 g .. + 4 of the lane's row
    if (nsplit == 1) {
        uint16_t* o = p.out + ((size_t)b * p.rows_total + grow) * kDv + 128 * wave + 4 * g;
#pragma unroll
        for (int t = 0; t < 8; ++t)
            *(u32x2*)(o + 16 * t) = u32x2{pack_bf16x2(v[t][0], v[t][1]), pack_bf16x2(v[t][2], v[t][3])};
    } else {
        float* o = p.part_o + ((size_t)slot * p.rows_total + grow) * kDv + 128 * wave + 4 * g;
#pragma unroll
        for (int t = 0; t < 8; ++t) *(f32x4*)(o + 16 * t) = v[t];
    }
    if (wave == 0 && g == 0) {
        const float lse = lt > 0.f ? (mall + __log2f(lt)) * kLn2 : -INFINITY;
        if (nsplit == 1) p.lse[(size_t)b * p.rows_total + grow] = lse;
        else p.part_lse[(size_t)slot * p.rows_total + grow] = lse;
    }
}

// ---------------------------------------------------------------- streaming kernel

constexpr int kMaxTopk = 2048;           // sparse decode: longest token list
constexpr int kRowTabB = kMaxTopk * 4;   // sparse decode: cache row of each listed token of the unit

// SPARSE: the unit's tokens are entries of a token list rather than a run of
// cache blocks (sparse decode). Before any copy the workgroup translates its
// list entries into cache row numbers (block_table[page] * 64 + row) in LDS,
// -1 for padding; a sub-tile's 16 rows are then copied from 16 unrelated
// places, padding rows from the unit's first listed row (finite data, masked).
template <int NR, bool SPARSE>
__global__ __launch_bounds__(256) void decode_stream_kernel(DecodeParams p)
{
    constexpr int R = 16 * NR;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kLdsA + (SPARSE ? kRowTabB : 0)];
    const unsigned lds0 = lds_base(smem);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int c16 = lane & 15;

    const i32x8 meta = sload8(p.meta + (size_t)blockIdx.x * kMetaInts);
    const int b = meta[0];
    const int j0 = meta[1];
    const int j1 = meta[3];
    const int L = meta[5];
    const int slot = meta[6];
    const int nsplit = meta[7];
    if (b >= p.batch || j0 >= j1) return;
    const int tok_begin = j0 * kPage;
    const int tok_end = SPARSE ? min(min(j1 * kPage, L), p.topk) : min(j1 * kPage, L);
    const int nsub = tok_end > tok_begin ? (tok_end - tok_begin + 15) >> 4 : 0;
    int K = nsub > wave ? (nsub - wave + 3) >> 2 : 0;         // this wave's sub-tiles: wave, wave+4, ...
    const int32_t* table = p.block_table + (size_t)b * p.max_blocks;
    const int npages = j1 - j0;
    const int page_vec = (!SPARSE && lane < npages && j0 + lane < p.max_blocks) ? table[j0 + lane] : 0;
    const unsigned rowtab = lds0 + kLdsA;                   // SPARSE: int32 per listed token of the unit
    int fallback = 0;                                       // SPARSE: cache row for padding entries
    if constexpr (SPARSE) {
        const int32_t* list = p.indices + (size_t)b * p.topk;
        const int32_t* rtable = p.block_table + (size_t)(b / p.sq_real) * p.max_blocks;
        // every list entry of the thread first, then every table entry they name: two
        // memory round trips in all rather than two per entry
        constexpr int kPer = kMaxTopk / 256;
        const int nent = tok_end - tok_begin;
        int t[kPer], pg[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int e = (int)threadIdx.x + 256 * j;
            t[j] = e < nent ? list[tok_begin + e] : -1;
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) pg[j] = (t[j] >= 0 && (t[j] >> 6) < p.max_blocks) ? rtable[t[j] >> 6] : -1;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int e = (int)threadIdx.x + 256 * j;
            const int rowid = (pg[j] >= 0 && (int64_t)pg[j] < p.nblocks) ? pg[j] * kPage + (t[j] & (kPage - 1)) : -1;
            if (e < nent) *(__attribute__((address_space(3))) int*)(uintptr_t)(rowtab + 4u * (unsigned)e) = rowid;
        }
        settle_loads();
        wg_barrier();
        fallback = -1;
        for (int c0 = 0; c0 < tok_end - tok_begin && fallback < 0; c0 += 64) {
            const int v = c0 + lane < tok_end - tok_begin
                              ? *(const __attribute__((address_space(3))) int*)(uintptr_t)(rowtab + 4u * (unsigned)(c0 + lane))
                              : -1;
            const unsigned long long any = __builtin_amdgcn_ballot_w64(v >= 0);
            if (any) fallback = __builtin_amdgcn_readlane(v, __builtin_ctzll(any));
        }
        if (fallback < 0) K = 0;                            // no listed token: an empty partial
    }

    float mrun[NR], lrun[NR];
    f32x4 acc[NR][32];
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
        mrun[rt] = -INFINITY;
        lrun[rt] = 0.f;
#pragma unroll
        for (int nt = 0; nt < 32; ++nt) acc[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const unsigned slot0 = lds0 + (unsigned)(2 * wave) * kSlotA;
    // lane offsets of the copies of a whole 16-row sub-tile (copy_rows' map with valid = 16);
    // SPARSE: the lane's byte offset within its row, and in bit i of `second` whether
    // the lane of copy i takes the copy's second row
    unsigned soff[kDmaA];
    unsigned second = 0;
#pragma unroll
    for (int i = 0; i < kDmaA; ++i) {
        const int q = i * 64 + lane;
        int r = (int)(__umul24((unsigned)q, 898u) >> 16);
        int c = q - kRowSlots * r;
        c = c < kChunks ? c : 0;
        if constexpr (SPARSE) {
            soff[i] = (unsigned)(c * 16);
            second |= (r != (i * 64) / kRowSlots ? 1u : 0u) << i;
        } else {
            r = r < 16 ? r : 0;
            soff[i] = (unsigned)(r * kRowBytes + c * 16);
        }
    }
    auto issue = [&](int k) {
        const int tok = tok_begin + 16 * (wave + 4 * k);
        if constexpr (SPARSE) {
            // lanes 0-15 fetch the cache rows of the sub-tile's 16 tokens (padding
            // and tokens past the list: the fallback row); copy i spans slot rows
            // r0 = 64 i / 73 and r0 + 1, whose bases are formed in scalar registers
            const unsigned dst = slot0 + (unsigned)(k & 1) * kSlotA;
            int rid = -1;
            if (lane < 16 && tok + lane < tok_end)
                rid = *(const __attribute__((address_space(3))) int*)(uintptr_t)(rowtab + 4u * (unsigned)(tok - tok_begin + lane));
            rid = rid >= 0 ? rid : fallback;
            const unsigned char* kc = (const unsigned char*)p.kcache;
#pragma unroll
            for (int i = 0; i < kDmaA; ++i) {
                const int r0 = (i * 64) / kRowSlots;
                const int r1 = r0 + 1 < 16 ? r0 + 1 : 0;             // slot positions past row 15: any real row
                const unsigned char* base0 = kc + (size_t)__builtin_amdgcn_readlane(rid, r0) * kRowBytes;
                const unsigned char* base1 = kc + (size_t)__builtin_amdgcn_readlane(rid, r1) * kRowBytes;
                dma16((((second >> i) & 1u) ? base1 : base0) + soff[i], dst + (unsigned)i * 1024u);
            }
            return;
        }
        const int pidx = (tok >> 6) - j0;
        const int page = safe_page(pidx < 64 ? __builtin_amdgcn_readlane(page_vec, pidx)
                                             : (j0 + pidx < p.max_blocks ? sload(table + j0 + pidx) : 0),
                                   p.nblocks);
        const unsigned char* gbase = (const unsigned char*)p.kcache + (size_t)page * kPageBytes +
                                     (size_t)(tok & 63) * kRowBytes;
        const unsigned dst = slot0 + (unsigned)(k & 1) * kSlotA;
        if (tok_end - tok >= 16) {
#pragma unroll
            for (int i = 0; i < kDmaA; ++i) dma16s(gbase, soff[i], dst + (unsigned)i * 1024u);
        } else {
            copy_rows(gbase, tok_end - tok, dst, 0, 1, kDmaA, lane);
        }
    };

    // Prologue. Every wave's first slot is issued first; the workgroup's 16
    // query rows are copied to LDS (into wave 3's second slot, padded rows like
    // the cache slots) by all four waves, so that no compiler-visible load has
    // to be awaited behind the block copies: each wave can start on its first
    // slot while its second is still in flight.
    static_assert(NR == 1, "one 16-row query tile per workgroup");
    const unsigned qslot = lds0 + 7u * kSlotA;
    const unsigned char* qbase = (const unsigned char*)(p.q + ((size_t)b * p.rows_total + blockIdx.y * R) * kDqk);
    settle_loads();                                         // page_vec: every later wait is for copies only
    if (K > 0) issue(0);
    copy_rows(qbase, R, qslot, wave, 4, kDmaA, lane);
    if (wave < 3 && K > 1) {
        issue(1);
        MLA_WAIT_VM(19);                                   // the slot-0 and query copies have landed
    } else {
        MLA_WAIT_VM(0);
    }
    wg_barrier();
    bf16x8 qf[NR][18];
    {
        const unsigned qa = qslot + (unsigned)(c16 * kLdsRow + 16 * g);
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) qf[0][ks] = __builtin_bit_cast(bf16x8, lds_load16(qa + 64 * ks));
        // the queries live in AGPRs, which the matrix ops read directly (left to the
        // register allocator they are parked there and copied back every step)
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) asm volatile("" : "+a"(qf[0][ks]));
    }
    wg_barrier();                                           // every wave holds its queries
    if (wave == 3 && K > 1) issue(1);
    int lim[NR];
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
        const int row = blockIdx.y * R + rt * 16 + c16;
        const int iq = row / p.h_q;
        lim[rt] = SPARSE ? tok_end : min(tok_end, p.causal ? L - (p.s_q - 1 - iq) : L);
    }

    const unsigned a_off = (unsigned)(stream_token(c16) * kLdsRow + g * 16);
    const unsigned v_off = (unsigned)(stream_token(4 * g + (c16 >> 2)) * kLdsRow + 8 * (c16 & 3));
    for (int k = 0; k < K; ++k) {
        if (k + 1 < K) MLA_WAIT_VM(19); else MLA_WAIT_VM(0);
        const unsigned sb = slot0 + (unsigned)(k & 1) * kSlotA;
        const int tok0 = tok_begin + 16 * (wave + 4 * k);

        // every LDS read of this slot up front: 18 K chunks (QK^T A operand) and
        // 32 transposed V pieces (PV A operand)
        s16x8 ka[18];
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) ka[ks] = lds_load16(sb + a_off + 64 * ks);
        s16x4 va[32];
#pragma unroll
        for (int nt = 0; nt < 32; ++nt) va[nt] = lds_tr4(sb + v_off + 32 * nt);
        // the slot's reads are done: refill it with sub-tile k + 2
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (k + 2 < K) issue(k + 2);

        // S^T = K Q^T for 16 tokens x R rows, two accumulation chains
        f32x4 s[NR];
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) {
            f32x4 e0 = {0.f, 0.f, 0.f, 0.f}, e1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 18; ks += 2) {
                e0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[ks]), qf[rt][ks], e0, 0, 0, 0);
                e1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[ks + 1]), qf[rt][ks + 1], e1, 0, 0, 0);
            }
            s[rt] = e0 + e1;
        }

        // scale, mask, online softmax; s[rt][i] is token tok0 + stream_token(4g + i)
        s16x4 pb[NR];
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) {
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = tok0 + stream_token(4 * g + i);
                bool vis = t < lim[rt];
                if constexpr (SPARSE)
                    vis = vis && *(const __attribute__((address_space(3))) int*)(uintptr_t)(rowtab + 4u * (unsigned)(t - tok_begin)) >= 0;
                const float v = vis ? s[rt][i] * p.scale_log2 : -INFINITY;
                s[rt][i] = v;
                tmax = fmaxf(tmax, v);
            }
            tmax = xor32_max(xor16_max(tmax));
            const bool need = tmax > mrun[rt] + kLazyTau;
            if (wave_any(need)) {
                const float mnew = need ? tmax : mrun[rt];
                const float alpha = need ? __builtin_amdgcn_exp2f(mrun[rt] - mnew) : 1.f;
                lrun[rt] *= alpha;
#pragma unroll
                for (int nt = 0; nt < 32; ++nt) acc[rt][nt] *= alpha;
                mrun[rt] = mnew;
            }
            const float muse = mrun[rt] == -INFINITY ? 0.f : mrun[rt];
            float pv[4], psum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pv[i] = __builtin_amdgcn_exp2f(s[rt][i] - muse);
                psum += pv[i];
            }
            pb[rt] = __builtin_bit_cast(s16x4, u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])});
            lrun[rt] += xor32_sum(xor16_sum(psum));
        }

        // O^T += V^T P^T
#pragma unroll
        for (int nt = 0; nt < 32; ++nt) {
#pragma unroll
            for (int rt = 0; rt < NR; ++rt) acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[nt], pb[rt], acc[rt][nt], 0, 0, 0);
        }
    }

    stream_merge_store(p, acc[0], mrun[0], lrun[0], lds0, slot0, wave, lane, b, slot, nsplit);
}

// ---------------------------------------------------------------- FP8 streaming kernel
//
// The streaming kernel over an FP8 cache (E4M3 codes, one float32 scale per
// cached row). A sub-tile is 32 tokens (32 x 576 code bytes: the same LDS
// footprint as 16 bf16 rows), so that the PV product can take 32 tokens per
// v_mfma_f32_16x16x32_bf16. Codes are turned into bf16 exactly (every E4M3
// value is a bf16 value) right before the matrix ops; the row scales are
// applied to the scores (S_t * scale_t) and to P (P_t * scale_t before PV), so
// they never touch the matrix operands.
//
// Slot layout (19 KB, 1216 chunks of 16 B): rows 0-15 at chunk 37 r, rows 16-31
// at 37 r + 1 (576 B of codes + one pad chunk; the extra chunk keeps rows r
// and r + 16 in different banks for the transpose reads), then the 32 row
// scales at chunk 1185. K rows are read 8 bytes per lane (ds_read_b64); V^T
// comes from ds_read_b64_tr_b8: in each 16-lane group, output lane j byte e is
// byte j % 8 of source lane 2e + j / 8, so source lane 2e + p reads dims
// [16 dt + 8 p, +8) of token T(G, e) and output lane j gets dim 16 dt + j of
// the 8 tokens T(G, 0..7) -- the A operand of the 16x16x32 product.

// token (0..31 within the sub-tile) of element e of a lane of group g in the
// S^T tiles / P^T operand: elements 0-3 are tile 0 rows 4g..4g+3, 4-7 tile 1
__device__ __forceinline__ int f8_token(int g, int e) { return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4); }

// Lane map of copy i of a slot: position pos = 64 i + lane holds chunk c of row
// r, where pp = pos minus the pad chunk before row 16, r = pp / 37 (exact as
// (pp * 1772) >> 16 for pp < 2367), c = pp mod 37; pad chunks and rows >= valid
// read the run's first chunk. The scale positions of the last copy get the
// byte offset of their four scales in the run's scale array instead.
__device__ __forceinline__ unsigned f8_stream_offset(int i, int lane, int valid)
{
    const int pos = i * 64 + lane;
    if (pos >= kF8Scale && pos < kF8Scale + 8) return (unsigned)(16 * (pos - kF8Scale));
    const int pp = pos - (pos >= kF8Row16 ? 1 : 0);
    int r = (int)(__umul24((unsigned)pp, 1772u) >> 16);
    const int c = pp - kF8Chunks * r;
    const bool data = pos != kF8Row16 - 1 && c < 36 && r < 32;
    r = r < valid ? r : 0;
    return data ? (unsigned)(r * kDqk + 16 * c) : 0u;
}

__global__ __launch_bounds__(256) void decode_stream_fp8_kernel(DecodeParams p)
{
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kLdsA];
    const unsigned lds0 = lds_base(smem);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int c16 = lane & 15;

    const i32x8 meta = sload8(p.meta + (size_t)blockIdx.x * kMetaInts);
    const int b = meta[0];
    const int j0 = meta[1];
    const int j1 = meta[3];
    const int L = meta[5];
    const int slot = meta[6];
    const int nsplit = meta[7];
    if (b >= p.batch || j0 >= j1) return;
    const int tok_begin = j0 * kPage;
    const int tok_end = min(j1 * kPage, L);
    const int nsub = (tok_end - tok_begin + 31) >> 5;
    const int K = nsub > wave ? (nsub - wave + 3) >> 2 : 0;   // this wave's sub-tiles: wave, wave+4, ...
    const int32_t* table = p.block_table + (size_t)b * p.max_blocks;
    const int npages = j1 - j0;
    const int page_vec = (lane < npages && j0 + lane < p.max_blocks) ? table[j0 + lane] : 0;
    const unsigned char* codes = (const unsigned char*)p.kcache;

    float mrun = -INFINITY, lrun = 0.f;
    f32x4 acc[32];
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const unsigned slot0 = lds0 + (unsigned)(2 * wave) * kSlotA;
    // lane offsets of the copies of a whole 32-row sub-tile; in the last copy the
    // lanes at the scale positions (fscl) take their offset from the run's scales
    unsigned foff[kDmaA];
#pragma unroll
    for (int i = 0; i < kDmaA; ++i) foff[i] = f8_stream_offset(i, lane, 32);
    const bool fscl = (kDmaA - 1) * 64 + lane >= kF8Scale && (kDmaA - 1) * 64 + lane < kF8Scale + 8;
    auto issue = [&](int k) {
        const int tok = tok_begin + 32 * (wave + 4 * k);
        const int pidx = (tok >> 6) - j0;
        const int page = safe_page(pidx < 64 ? __builtin_amdgcn_readlane(page_vec, pidx)
                                             : (j0 + pidx < p.max_blocks ? sload(table + j0 + pidx) : 0),
                                   p.nblocks);
        const size_t row0 = (size_t)page * kPage + (size_t)(tok & 63);
        const unsigned char* gbase = codes + row0 * kDqk;
        const unsigned char* sbase = (const unsigned char*)(p.kscale + row0);
        const int valid = min(32, tok_end - tok);
        const unsigned dst = slot0 + (unsigned)(k & 1) * kSlotA;
        if (valid == 32) {
#pragma unroll
            for (int i = 0; i < kDmaA - 1; ++i) dma16s(gbase, foff[i], dst + (unsigned)i * 1024u);
            dma16(fscl ? sbase + foff[kDmaA - 1] : gbase + foff[kDmaA - 1], dst + (unsigned)(kDmaA - 1) * 1024u);
            return;
        }
#pragma unroll
        for (int i = 0; i < kDmaA; ++i) {
            const unsigned off = f8_stream_offset(i, lane, valid);
            if (i == kDmaA - 1)
                dma16(fscl ? sbase + off : gbase + off, dst + (unsigned)i * 1024u);
            else
                dma16s(gbase, off, dst + (unsigned)i * 1024u);
        }
    };

    // Prologue (as in the bf16 streaming kernel): the queries go through LDS
    // (wave 3's second slot), so that every later wait is for copies only.
    const unsigned qslot = lds0 + 7u * kSlotA;
    const unsigned char* qbase = (const unsigned char*)(p.q + ((size_t)b * p.rows_total + blockIdx.y * 16) * kDqk);
    settle_loads();
    if (K > 0) issue(0);
    copy_rows(qbase, 16, qslot, wave, 4, kDmaA, lane);
    if (wave < 3 && K > 1) {
        issue(1);
        MLA_WAIT_VM(19);
    } else {
        MLA_WAIT_VM(0);
    }
    wg_barrier();
    bf16x8 qf[18];
    {
        const unsigned qa = qslot + (unsigned)(c16 * kLdsRow + 16 * g);
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, lds_load16(qa + 64 * ks));
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) asm volatile("" : "+a"(qf[ks]));       // in AGPRs, as above
    }
    wg_barrier();
    if (wave == 3 && K > 1) issue(1);
    const int row = blockIdx.y * 16 + c16;
    const int iq = row / p.h_q;
    const int lim = min(tok_end, p.causal ? L - (p.s_q - 1 - iq) : L);

    // per-lane LDS offsets: K rows 16 hh + c16 at byte 8 g; V^T source row T(g, c16 / 2) at byte 8 (c16 % 2)
    const unsigned k_off0 = f8_row(c16) + 8u * (unsigned)g;
    const unsigned k_off1 = f8_row(16 + c16) + 8u * (unsigned)g;
    const unsigned v_off = f8_row(f8_token(g, c16 >> 1)) + 8u * (unsigned)(c16 & 1);
    for (int k = 0; k < K; ++k) {
        if (k + 1 < K) MLA_WAIT_VM(19); else MLA_WAIT_VM(0);
        const unsigned sb = slot0 + (unsigned)(k & 1) * kSlotA;
        const int tok0 = tok_begin + 32 * (wave + 4 * k);

        // the V^T operands and the row scales up front; K rows streamed through
        // QK^T (four k-steps ahead); the slot is refilled once QK^T has read it
        u32x2 vr[32];
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) {
            const auto t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) i32x2*)(uintptr_t)(sb + v_off + 16u * dt));
            vr[dt] = u32x2{(unsigned)t[0], (unsigned)t[1]};
        }
        const f32x4 sc0 = *(const lds_f32x4*)(uintptr_t)(sb + 16u * kF8Scale + 16u * g);
        const f32x4 sc1 = *(const lds_f32x4*)(uintptr_t)(sb + 16u * kF8Scale + 64u + 16u * g);

        // S^T = K Q^T for the two 16-token halves (k-step kk: half kk / 18, step kk % 18)
        auto kread = [&](int kk) {
            const unsigned off = (kk < 18 ? k_off0 : k_off1) + 32u * (unsigned)(kk % 18);
            return *(const __attribute__((address_space(3))) u32x2*)(uintptr_t)(sb + off);
        };
        f32x4 s[2];
        {
            // K fragments are read four k-steps ahead and converted one step ahead
            // (ping-pong), under the previous matrix op; a scheduling barrier per
            // step keeps that order (left alone, the compiler paired the reads and
            // waited for each pair two matrix ops after issuing it)
            u32x2 kr[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) kr[kk] = kread(kk);
            f32x4 e[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            bf16x8 a2[2];
            a2[0] = e4m3x8_to_bf16(kr[0]);
#pragma unroll
            for (int kk = 0; kk < 36; ++kk) {
                __builtin_amdgcn_sched_barrier(0);
                const int hh = kk / 18, ks = kk % 18;
                e[2 * hh + (ks & 1)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2[kk & 1], qf[ks], e[2 * hh + (ks & 1)],
                                                                            0, 0, 0);
                if (kk + 1 < 36) a2[(kk + 1) & 1] = e4m3x8_to_bf16(kr[(kk + 1) & 3]);
                if (kk + 4 < 36) kr[kk & 3] = kread(kk + 4);
            }
            __builtin_amdgcn_sched_barrier(0);
            s[0] = e[0] + e[1];
            s[1] = e[2] + e[3];
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (k + 2 < K) issue(k + 2);

        // row scales, mask, online softmax
        float sv[8], scu[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float sc = e < 4 ? sc0[e] : sc1[e - 4];
            const int t = tok0 + f8_token(g, e);
            const bool vis = t < lim;
            sv[e] = vis ? s[e >> 2][e & 3] * sc * p.scale_log2 : -INFINITY;
            scu[e] = vis ? sc : 0.f;                           // scales of rows past the end may be anything
        }
        float tmax = sv[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, sv[e]);
        tmax = xor32_max(xor16_max(tmax));
        const bool need = tmax > mrun + kLazyTau;
        if (wave_any(need)) {
            const float mnew = need ? tmax : mrun;
            const float alpha = need ? __builtin_amdgcn_exp2f(mrun - mnew) : 1.f;
            lrun *= alpha;
#pragma unroll
            for (int nt = 0; nt < 32; ++nt) acc[nt] *= alpha;
            mrun = mnew;
        }
        const float muse = mrun == -INFINITY ? 0.f : mrun;
        float pv[8], psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pe = __builtin_amdgcn_exp2f(sv[e] - muse);
            psum += pe;
            pv[e] = pe * scu[e];
        }
        lrun += xor32_sum(xor16_sum(psum));
        const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                                           pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])});

        // O^T += V^T (P scale)^T, 32 tokens per matrix op
#pragma unroll
        for (int nt = 0; nt < 32; ++nt)
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(vr[nt]), pb, acc[nt], 0, 0, 0);
    }

    stream_merge_store(p, acc, mrun, lrun, lds0, slot0, wave, lane, b, slot, nsplit);
}

hipError_t launch_decode_fp8(const DecodeParams& p, int num_units, int head_groups, int rows_wg, hipStream_t stream)
{
    dim3 grid(num_units, head_groups);
    switch (rows_wg) {
    case 16: hipLaunchKernelGGL(decode_stream_fp8_kernel, grid, dim3(256), 0, stream, p); break;
    case 64: return launch_wide_fp8(p, grid, stream);
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- split combine

// Merge split partials by their log-sum-exp: out = sum_k exp(lse_k - L) o_k,
// lse = L = log sum_k exp(lse_k). One thread per 4 dims of one (sequence, row);
// the partials are read U at a time (their lse and o loads issued together)
// and folded in with a running max. Sequences with no block get out = 0,
// lse = -inf; unsplit ones were written by the decode kernel.
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p)
{
    constexpr int U = 16;                                   // partials in flight per thread
    const int t = threadIdx.x & 127;                        // 4-dim chunk of the row
    const int row = blockIdx.x * 2 + (threadIdx.x >> 7);
    const int b = blockIdx.y;
    if (row >= p.rows_total) return;
    const int s0 = p.splits[b];
    const int ns = p.splits[b + 1] - s0;
    if (ns == 1) return;
    uint16_t* o = p.out + ((size_t)b * p.rows_total + row) * kDv + 4 * t;
    float* lo = p.lse + (size_t)b * p.rows_total + row;
    const float* lse_col = p.part_lse + (size_t)s0 * p.rows_total + row;
    const float* o_col = p.part_o + ((size_t)s0 * p.rows_total + row) * kDv + 4 * t;
    float m = -INFINITY, l = 0.f;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < ns; k += U) {
        float w[U];
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            w[u] = -INFINITY;
            v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (k + u < ns) {
                w[u] = lse_col[(size_t)(k + u) * p.rows_total];
                v[u] = *(const f32x4*)(o_col + (size_t)(k + u) * p.rows_total * kDv);
            }
        }
        float mk = m;
#pragma unroll
        for (int u = 0; u < U; ++u) mk = fmaxf(mk, w[u]);
        if (mk == -INFINITY) continue;                      // nothing visible yet
        const float sc = __expf(m - mk);                    // 0 while m is -inf
        l *= sc;
        a *= sc;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float e = __expf(w[u] - mk);
            l += e;
            a += v[u] * e;
        }
        m = mk;
    }
    if (m == -INFINITY) {
        *(ushort4*)o = make_ushort4(0, 0, 0, 0);
        if (t == 0) *lo = -INFINITY;
        return;
    }
    const float inv = 1.f / l;
    u32x2 r;
    r[0] = pack_bf16x2(a[0] * inv, a[1] * inv);
    r[1] = pack_bf16x2(a[2] * inv, a[3] * inv);
    *(u32x2*)o = r;
    if (t == 0) *lo = m + __logf(l);
}

// The combine for plans of 64-row workgroups, whose sequences have few splits
// (two or three in the 64-row workloads): one wave per two rows, lane l merges
// dims [8 l, 8 l + 8) of both rows, every partial of a pass in flight at once;
// the partials' log-sum-exps are wave-uniform (scalar loads). The merge is
// combine_kernel's, in passes of 8 partials instead of 16 (the same arithmetic
// up to 8 splits). (With 16-row plans, whose sequences have up to dozens of
// splits over few rows, this shape leaves too few waves in flight; they keep
// combine_kernel.)
__global__ __launch_bounds__(256) void combine_rows_kernel(CombineParams p)
{
    constexpr int U = 8;                                    // partials per pass
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b = blockIdx.y;
    const int s0 = cload(p.splits + b);
    const int ns = cload(p.splits + b + 1) - s0;
    if (ns == 1) return;
    const int row0 = (blockIdx.x * 4 + wave) * 2;
    if (row0 >= p.rows_total) return;
    const bool two = row0 + 1 < p.rows_total;
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    f32x4 a[2][2] = {};
    const float* lse_col = p.part_lse + (size_t)s0 * p.rows_total + row0;
    const float* o_col = p.part_o + ((size_t)s0 * p.rows_total + row0) * kDv + 8 * lane;
    for (int k = 0; k < ns; k += U) {
        float w[2][U];
        f32x4 v[2][U][2];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                w[r][u] = -INFINITY;
                v[r][u][0] = v[r][u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (k + u < ns && (r == 0 || two)) {
                    w[r][u] = *(const __attribute__((address_space(4))) float*)(uintptr_t)(lse_col + (size_t)(k + u) * p.rows_total + r);
                    const float* src = o_col + ((size_t)(k + u) * p.rows_total + r) * kDv;
                    v[r][u][0] = *(const f32x4*)src;
                    v[r][u][1] = *(const f32x4*)(src + 4);
                }
            }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            float mk = m[r];
#pragma unroll
            for (int u = 0; u < U; ++u) mk = fmaxf(mk, w[r][u]);
            if (mk == -INFINITY) continue;                  // nothing visible yet
            const float sc = __expf(m[r] - mk);             // 0 while m is -inf
            l[r] *= sc;
            a[r][0] *= sc;
            a[r][1] *= sc;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float e = __expf(w[r][u] - mk);
                l[r] += e;
                a[r][0] += v[r][u][0] * e;
                a[r][1] += v[r][u][1] * e;
            }
            m[r] = mk;
        }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        if (r == 1 && !two) break;
        const int row = row0 + r;
        uint16_t* o = p.out + ((size_t)b * p.rows_total + row) * kDv + 8 * lane;
        float* lo = p.lse + (size_t)b * p.rows_total + row;
        if (m[r] == -INFINITY) {
            *(u32x4*)o = u32x4{0u, 0u, 0u, 0u};
            if (lane == 0) *lo = -INFINITY;
            continue;
        }
        const float inv = 1.f / l[r];
        u32x4 q;
        q[0] = pack_bf16x2(a[r][0][0] * inv, a[r][0][1] * inv);
        q[1] = pack_bf16x2(a[r][0][2] * inv, a[r][0][3] * inv);
        q[2] = pack_bf16x2(a[r][1][0] * inv, a[r][1][1] * inv);
        q[3] = pack_bf16x2(a[r][1][2] * inv, a[r][1][3] * inv);
        *(u32x4*)o = q;
        if (lane == 0) *lo = m[r] + __logf(l[r]);
    }
}

hipError_t launch_decode(const DecodeParams& p, int num_units, int head_groups, int rows_wg, hipStream_t stream)
{
    dim3 grid(num_units, head_groups);
    switch (rows_wg) {
    case 16: hipLaunchKernelGGL((decode_stream_kernel<1, false>), grid, dim3(256), 0, stream, p); break;
    case 64: return launch_wide(p, grid, stream);
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_sparse(const DecodeParams& p, int num_units, int head_groups, hipStream_t stream)
{
    dim3 grid(num_units, head_groups);
    hipLaunchKernelGGL((decode_stream_kernel<1, true>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream)
{
    if (p.rows_total % 64 == 0) {
        hipLaunchKernelGGL(combine_rows_kernel, dim3((p.rows_total + 7) / 8, p.batch), dim3(256), 0, stream, p);
    } else {
        hipLaunchKernelGGL(combine_kernel, dim3((p.rows_total + 1) / 2, p.batch), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace mla
