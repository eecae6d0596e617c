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
//  * Wide kernel (64 query rows): two row groups of 32, each split over two
//    waves (QK^T by column halves, PV by output-dim halves), share a ring of
//    four 32-token LDS slots (three in flight while one is used); QK^T and PV
//    on v_mfma_f32_32x32x16_bf16. A unit may cover several sequences.
//
// Data path common to both:
//  * a cache block is 64 contiguous rows of 1152 B; in the streaming kernel an
//    LDS row is 72 chunks of 16 B plus one pad chunk (stride 1168 B), in the
//    wide kernel it is unpadded with chunk c of row r stored at c ^ (r % 8);
//  * S^T = K Q^T: K rows are the MFMA A operand (ds_read_b128), Q^T the B
//    operand held in VGPRs. The S^T accumulator layout (lane = query row,
//    4 tokens per element group) is exactly the P^T B operand of O^T = V^T P^T,
//    so P never leaves registers;
//  * V^T comes from ds_read_b64_tr_b16: within each 16-lane group, output lane
//    j element e is element j%4 of what source lane 4e + j/4 read, so source
//    lanes read 4 dims of 4 token rows and every output lane ends with one dim
//    of 4 tokens -- the MFMA A operand;
//  * the MFMA row <-> token map is permuted, token(a) = 8(a/8) + 2(a%4) + (a/4)%2,
//    so that 8 consecutive A rows hit 8 different 16-byte bank groups and the 4
//    rows a transpose read combines hit 4 different 32-byte bank groups;
//  * scores are scaled into the exp2 domain; the running max is raised (and O
//    rescaled) only when a score exceeds it by more than 2^8, so P <= 256;
//  * rows past the end of a sequence are loaded from the block's first valid
//    row instead (finite data, masked to p = 0), so no LDS row holds garbage;
//  * block-table entries and scalars are read with scalar loads so that they
//    never wait on the vector-memory counter that tracks the block copies.
#include "mla_common.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) s16x8 lds_s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_rw;

constexpr int kLdsRow = 1168;            // LDS row stride: 72 data chunks + 1 pad chunk of 16 B
constexpr int kRowSlots = 73;
constexpr int kChunks = 72;
constexpr float kLazyTau = 8.f;          // exp2-domain slack of the running max
constexpr float kLn2 = 0.69314718055994531f;

// ---------------------------------------------------------------- primitives

// One 16-byte global->LDS copy per lane. lds_addr (uniform) is the LDS byte
// address of the wave's 1 KB destination; lane l lands at lds_addr + 16 l.
// Issued through asm so the compiler does not order later LDS reads of other
// buffers behind it; completion is awaited explicitly with vmcnt.
__device__ __forceinline__ void dma16(const unsigned char* gptr, unsigned lds_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(lds_addr)
                 : "memory");
}

#define MLA_WAIT_VM(n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")

// vmcnt(0) issued through the builtin, which the compiler's own wait-count
// tracking sees: after it, loads the compiler issued (queries, table rows) are
// known complete, so it inserts no waits for them inside the copy pipeline
// (such a wait would also stall on every block copy in flight).
__device__ __forceinline__ void settle_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ void wg_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Scalar load of a wave-uniform int (waits for it in the same asm block).
__device__ __forceinline__ int sload(const int32_t* ptr)
{
    int v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
    return v;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Scalar load of 8 consecutive wave-uniform ints (one plan row).
__device__ __forceinline__ i32x8 sload8(const int32_t* ptr)
{
    i32x8 v;
    asm volatile("s_load_dwordx8 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
    return v;
}

// Reductions across the lanes l, l^16, l^32, l^48 (one value per 16-lane row)
// with the gfx950 lane-swap instructions: each swap exchanges whole 16- or
// 32-lane halves between two operands, so combining both results pairs every
// lane with its partner.
__device__ __forceinline__ float xor32_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ unsigned lds_base(unsigned char* smem)
{
    return (unsigned)(uintptr_t)(lds_u8*)smem;
}

__device__ __forceinline__ s16x8 lds_load16(unsigned addr) { return *(const lds_s16x8*)(uintptr_t)addr; }

__device__ __forceinline__ s16x4 lds_tr4(unsigned addr)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)addr);
}

__device__ __forceinline__ int token_of_row(int a) { return ((a >> 3) << 3) + ((a & 3) << 1) + ((a >> 2) & 1); }

__device__ __forceinline__ unsigned short bf16_rne(float f)
{
    unsigned u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (unsigned short)(u >> 16);
}

__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

// Copy rows [0, 16 or 32) of a block run starting at gbase (valid of them real)
// into an LDS slot; copies first, first+step, ... < ninstr of 1 KB each.
__device__ __forceinline__ void copy_rows(const unsigned char* gbase, int valid, unsigned slot, int first,
                                          int step, int ninstr, int lane)
{
    for (int i = first; i < ninstr; i += step) {
        const int q = i * 64 + lane;
        int r = q / kRowSlots;
        int c = q - r * kRowSlots;
        r = r < valid ? r : 0;
        c = c < kChunks ? c : 0;
        dma16(gbase + r * kRowBytes + c * 16, slot + (unsigned)i * 1024u);
    }
}

// ---------------------------------------------------------------- streaming kernel

constexpr int kSlotA = 19 * 1024;        // 16 rows x 1168 B, rounded up to whole 1 KB copies
constexpr int kDmaA = 19;
constexpr int kLdsA = 8 * kSlotA;        // two slots per wave: 155,648 B

template <int NR>
__global__ __launch_bounds__(256) void decode_stream_kernel(DecodeParams p)
{
    constexpr int R = 16 * NR;
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
    const int nsub = (tok_end - tok_begin + 15) >> 4;
    const int K = nsub > wave ? (nsub - wave + 3) >> 2 : 0;   // this wave's sub-tiles: wave, wave+4, ...
    const int32_t* table = p.block_table + (size_t)b * p.max_blocks;
    const int npages = j1 - j0;
    const int page_vec = lane < npages ? table[j0 + lane] : 0;

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
    auto issue = [&](int k) {
        const int tok = tok_begin + 16 * (wave + 4 * k);
        const int pidx = (tok >> 6) - j0;
        const int page = pidx < 64 ? __builtin_amdgcn_readlane(page_vec, pidx) : sload(table + j0 + pidx);
        const unsigned char* gbase = (const unsigned char*)p.kcache + (size_t)page * kPageBytes +
                                     (size_t)(tok & 63) * kRowBytes;
        copy_rows(gbase, min(16, tok_end - tok), slot0 + (unsigned)(k & 1) * kSlotA, 0, 1, kDmaA, lane);
    };

    if (K > 0) issue(0);
    if (K > 1) issue(1);

    // queries (issued after the first copies; the settle below waits for both)
    bf16x8 qf[NR][18];
    int lim[NR];
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
        const int row = blockIdx.y * R + rt * 16 + c16;
        const uint16_t* qrow = p.q + ((size_t)b * p.rows_total + row) * kDqk + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) qf[rt][ks] = __builtin_bit_cast(bf16x8, *(const s16x8*)(qrow + 32 * ks));
        const int iq = row / p.h_q;
        lim[rt] = min(tok_end, p.causal ? L - (p.s_q - 1 - iq) : L);
    }
    settle_loads();


    const unsigned a_off = (unsigned)(token_of_row(c16) * kLdsRow + g * 16);
    const unsigned v_off = (unsigned)(token_of_row(4 * g + (c16 >> 2)) * kLdsRow + 8 * (c16 & 3));
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

        // the slot's reads are done: refill it with sub-tile k + 2
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (k + 2 < K) issue(k + 2);

        // scale, mask, online softmax; s[rt][i] is token tok0 + token_of_row(4g + i)
        s16x4 pb[NR];
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) {
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = tok0 + token_of_row(4 * g + i);
                const float v = (t < lim[rt]) ? s[rt][i] * p.scale_log2 : -INFINITY;
                s[rt][i] = v;
                tmax = fmaxf(tmax, v);
            }
            tmax = xor32_max(xor16_max(tmax));
            const bool need = tmax > mrun[rt] + kLazyTau;
            if (wave_any(need)) {
                const float mnew = need ? tmax : mrun[rt];
                const float alpha = need ? exp2f(mrun[rt] - mnew) : 1.f;
                lrun[rt] *= alpha;
#pragma unroll
                for (int nt = 0; nt < 32; ++nt) acc[rt][nt] *= alpha;
                mrun[rt] = mnew;
            }
            const float muse = mrun[rt] == -INFINITY ? 0.f : mrun[rt];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = exp2f(s[rt][i] - muse);
                psum += pv;
                pb[rt][i] = (short)bf16_rne(pv);
            }
            lrun[rt] += xor32_sum(xor16_sum(psum));
        }

        // O^T += V^T P^T
#pragma unroll
        for (int nt = 0; nt < 32; ++nt) {
#pragma unroll
            for (int rt = 0; rt < NR; ++rt) acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[nt], pb[rt], acc[rt][nt], 0, 0, 0);
        }
    }

    // ---- merge the four waves' (m, l, O) and write the result. Wave w owns
    // output tiles nt in [8w, 8w + 8) (dims [128w, 128w + 128)) and keeps them
    // in registers; it posts its other 24 tiles to LDS as bf16 (unscaled) for
    // their owners, and its running max/sum for every row.
    wg_barrier();                                            // every wave is done with its slots
    lds_f32* stat_m = (lds_f32*)(uintptr_t)lds0;            // [4][R]
    lds_f32* stat_l = stat_m + 4 * R;                         // [4][R]
    const unsigned xbuf = lds0 + 1024;                       // [4][NR][32 tiles][64 lanes] x 8 B
    if (g == 0) {
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) {
            stat_m[wave * R + rt * 16 + c16] = mrun[rt];
            stat_l[wave * R + rt * 16 + c16] = lrun[rt];
        }
    }
#pragma unroll
    for (int rt = 0; rt < NR; ++rt)
#pragma unroll
        for (int nt = 0; nt < 32; ++nt) {
            if ((nt >> 3) == wave) continue;
            s16x4 v;
            v[0] = (short)bf16_rne(acc[rt][nt][0]);
            v[1] = (short)bf16_rne(acc[rt][nt][1]);
            v[2] = (short)bf16_rne(acc[rt][nt][2]);
            v[3] = (short)bf16_rne(acc[rt][nt][3]);
            *(lds_s16x4_rw*)(uintptr_t)(xbuf + (unsigned)((((wave * NR + rt) * 32 + nt) * 64 + lane) * 8)) = v;
        }
    wg_barrier();
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
        const int rrow = rt * 16 + c16;
        float mw[4], mall = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            mw[w] = stat_m[w * R + rrow];
            mall = fmaxf(mall, mw[w]);
        }
        float fw[4], lt = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            fw[w] = mw[w] == -INFINITY ? 0.f : exp2f(mw[w] - mall);
            lt += stat_l[w * R + rrow] * fw[w];
        }
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const int grow = blockIdx.y * R + rrow;
#pragma unroll
        for (int nt = 0; nt < 32; ++nt) {
            if ((nt >> 3) != wave) continue;                  // static tile index, uniform branch
            f32x4 v = acc[rt][nt] * fw[nt >> 3];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if (w == wave) continue;
                const s16x4 o = *(const lds_s16x4_rw*)(uintptr_t)(
                    xbuf + (unsigned)((((w * NR + rt) * 32 + nt) * 64 + lane) * 8));
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] += __uint_as_float((unsigned)(unsigned short)o[i] << 16) * fw[w];
            }
            v *= inv;
            const int d = 16 * nt + 4 * g;
            if (nsplit == 1) {
                ushort4 ob;
                ob.x = bf16_rne(v[0]); ob.y = bf16_rne(v[1]); ob.z = bf16_rne(v[2]); ob.w = bf16_rne(v[3]);
                *(ushort4*)(p.out + ((size_t)b * p.rows_total + grow) * kDv + d) = ob;
            } else {
                *(f32x4*)(p.part_o + ((size_t)slot * p.rows_total + grow) * kDv + d) = v;
            }
        }
        if (wave == 0 && g == 0) {
            const float lse = lt > 0.f ? (mall + __log2f(lt)) * kLn2 : -INFINITY;
            if (nsplit == 1) p.lse[(size_t)b * p.rows_total + grow] = lse;
            else p.part_lse[(size_t)slot * p.rows_total + grow] = lse;
        }
    }
}

// ---------------------------------------------------------------- wide kernel
//
// 64 query rows per workgroup, four waves: wave = 2 rg + kh holds rows
// [32 rg, 32 rg + 32) of the workgroup; kh picks the half of the work it does.
// QK^T: wave kh contracts cached columns [288 kh, 288 kh + 288) (its 72-register
// half of Q); the two partial S^T tiles of a row group are summed through LDS.
// PV: wave kh accumulates output dims [256 kh, 256 kh + 256) (128 registers).
// Both waves of a row group run the same softmax on the same S and so keep
// identical running max and sum. The four waves share a ring of four 32-token
// slots (three in flight while one is used). Slots hold rows of 1152 B with
// chunk c of row r at position c ^ (r % 8), which with the token permutation
// keeps b128 and transpose reads conflict free.

constexpr int kSlotB = 32 * kRowBytes;   // 36,864 B = 36 copies of 1 KB
constexpr int kDmaB = 36;                // 9 per wave
constexpr int kXbufB = 4 * 4096;         // partial S^T tiles, 4 KB per wave
constexpr int kLdsB = 4 * kSlotB + kXbufB;   // 163,840 B

// The run of sequence b inside a unit: tokens [tb, te) of a sequence of L tokens.
struct Segment {
    int b, tb, te, L;
};

__device__ __forceinline__ Segment unit_segment(const DecodeParams& p, int b, int b0, int j0, int b1, int j1)
{
    Segment s;
    s.b = b;
    s.L = sload(p.seqlens + b);
    const int nb = blocks_of(s.L);
    s.tb = (b == b0 ? j0 : 0) * kPage;
    const int je = (b == b1) ? j1 : nb;
    s.te = min(je * kPage, s.L);
    return s;
}

// First non-empty segment of the unit at or after sequence b (b = batch when none).
__device__ __forceinline__ Segment next_segment(const DecodeParams& p, int b, int b0, int j0, int b1, int j1)
{
    for (; b <= b1 && b < p.batch; ++b) {
        Segment s = unit_segment(p, b, b0, j0, b1, j1);
        if (s.tb < s.te) return s;
    }
    Segment none;
    none.b = p.batch; none.tb = 0; none.te = 0; none.L = 0;
    return none;
}

// LDS byte offset of chunk c of row r in a swizzled slot.
__device__ __forceinline__ unsigned swz(int r, int c) { return (unsigned)(r * kRowBytes + ((c ^ (r & 7)) << 4)); }

__global__ __launch_bounds__(256) void decode_wide_kernel(DecodeParams p)
{
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kLdsB];
    const unsigned lds0 = lds_base(smem);
    const unsigned xbuf = lds0 + 4 * kSlotB;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = wave >> 1;
    const int kh = wave & 1;
    const int h = lane >> 5;
    const int r32 = lane & 31;
    const int i16 = lane & 15;
    const int dh = (lane >> 4) & 1;

    const i32x8 meta = sload8(p.meta + (size_t)blockIdx.x * kMetaInts);
    const int b0 = meta[0];
    const int j0 = meta[1];
    const int b1 = meta[2];
    const int j1 = meta[3];
    const int first_slot = meta[6];

    const int row = blockIdx.y * 64 + 32 * rg + r32;        // this lane's query row
    const int iq = row / p.h_q;

    Segment is = next_segment(p, b0, b0, j0, b1, j1);      // issue cursor
    if (is.b >= p.batch) return;
    int itok = is.tb;
    int ipage_idx = -1, ipage = 0;
    Segment cs = is;                                        // compute cursor

    // copy slot n: this wave's 9 of its 36 1 KB copies; lane l of copy i fills
    // LDS position s of row r (72 r + s = 64 i + l) with chunk s ^ (r % 8)
    auto issue = [&](int n) {
        const int pidx = itok >> 6;
        if (pidx != ipage_idx) {
            ipage = sload(p.block_table + (size_t)is.b * p.max_blocks + pidx);
            ipage_idx = pidx;
        }
        const unsigned char* gbase = (const unsigned char*)p.kcache + (size_t)ipage * kPageBytes +
                                     (size_t)(itok & 63) * kRowBytes;
        const int valid = min(32, is.te - itok);
        const unsigned slot = lds0 + (unsigned)(n & 3) * kSlotB;
#pragma unroll
        for (int k = 0; k < kDmaB / 4; ++k) {
            const int i = wave + 4 * k;
            const int q = i * 64 + lane;
            const int r = q / kChunks;
            const int c = (q - r * kChunks) ^ (r & 7);
            dma16(gbase + (r < valid ? r : 0) * kRowBytes + c * 16, slot + (unsigned)i * 1024u);
        }
        itok += 32;
        if (itok >= is.te) {
            is = next_segment(p, is.b + 1, b0, j0, b1, j1);
            itok = is.tb;
            ipage_idx = -1;
        }
    };

    int n_issued = 0;
    for (int k = 0; k < 3 && is.b < p.batch; ++k) issue(n_issued++);

    // QK^T A operand: token row tokA = token_of_row(r32), chunk 36 kh + 2 ks + h
    const int tokA = token_of_row(r32);
    // PV A operand (transposed V): source row token_of_row(16 kp + 8 half + 4h + i16/4),
    // dims 256 kh + 32 nt + 16 dh + 4 (i16 % 4), i.e. chunk 32 kh + 4 nt + 2 dh + (i16 % 4)/2
    unsigned v_off[2][2][2];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int par = 0; par < 2; ++par) {
                const int r = token_of_row(16 * kp + 8 * half + 4 * h + (i16 >> 2));
                const int c = 32 * kh + 4 * par + 2 * dh + ((i16 & 3) >> 1);
                v_off[kp][half][par] = swz(r, c) + 8u * (unsigned)(i16 & 1);
            }

    int n = 0;                                              // slot being computed
    while (cs.b < p.batch) {
        // new segment: this wave's half of its 32 query rows, fresh softmax state
        bf16x8 qf[18];
        {
            const uint16_t* qrow = p.q + ((size_t)cs.b * p.rows_total + row) * kDqk + 288 * kh + 8 * h;
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, *(const s16x8*)(qrow + 16 * ks));
            settle_loads();
        }
        f32x16 acc[8];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[nt][i] = 0.f;
        float mrun = -INFINITY, lrun = 0.f;
        const int lim = min(cs.te, p.causal ? cs.L - (p.s_q - 1 - iq) : cs.L);

        for (int ctok = cs.tb; ctok < cs.te; ctok += 32, ++n) {
            const int later = n_issued - 1 - n;
            if (later <= 0) MLA_WAIT_VM(0);
            else if (later == 1) MLA_WAIT_VM(9);
            else MLA_WAIT_VM(18);
            wg_barrier();
            // the buffer of slot n-1 is free: every wave has passed the barrier
            if (is.b < p.batch) issue(n_issued++);
            const unsigned sb = lds0 + (unsigned)(n & 3) * kSlotB;

            // partial S^T over this wave's half of the columns, two accumulators
            f32x16 s0, s1;
#pragma unroll
            for (int i = 0; i < 16; ++i) { s0[i] = 0.f; s1[i] = 0.f; }
#pragma unroll
            for (int ks = 0; ks < 18; ks += 2) {
                const s16x8 k0 = lds_load16(sb + swz(tokA, 36 * kh + 2 * ks + h));
                const s16x8 k1 = lds_load16(sb + swz(tokA, 36 * kh + 2 * ks + 2 + h));
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k0), qf[ks], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k1), qf[ks + 1], s1, 0, 0, 0);
            }
            s0 += s1;
            {
                const unsigned mine = xbuf + (unsigned)(wave * 4096 + lane * 64);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *(lds_f32x4*)(uintptr_t)(mine + 16 * j) = f32x4{s0[4 * j], s0[4 * j + 1], s0[4 * j + 2], s0[4 * j + 3]};
            }
            wg_barrier();
            {
                const unsigned other = xbuf + (unsigned)((wave ^ 1) * 4096 + lane * 64);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 o = *(const lds_f32x4*)(uintptr_t)(other + 16 * j);
                    s0[4 * j] += o[0]; s0[4 * j + 1] += o[1]; s0[4 * j + 2] += o[2]; s0[4 * j + 3] += o[3];
                }
            }

            // element i of S^T is token ctok + token_of_row(8(i/4) + 4h + i%4) of query row r32
            float sv[16];
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int t = ctok + token_of_row(8 * (i >> 2) + 4 * h + (i & 3));
                const float v = (t < lim) ? s0[i] * p.scale_log2 : -INFINITY;
                sv[i] = v;
                tmax = fmaxf(tmax, v);
            }
            tmax = xor32_max(tmax);
            const bool need = tmax > mrun + kLazyTau;
            if (wave_any(need)) {
                const float mnew = need ? tmax : mrun;
                const float alpha = need ? exp2f(mrun - mnew) : 1.f;
                lrun *= alpha;
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) acc[nt] *= alpha;
                mrun = mnew;
            }
            const float muse = mrun == -INFINITY ? 0.f : mrun;
            float psum = 0.f;
            s16x8 pb[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pv = exp2f(sv[i] - muse);
                psum += pv;
                pb[i >> 3][i & 7] = (short)bf16_rne(pv);
            }
            lrun += xor32_sum(psum);

            // O^T += V^T P^T over two 16-token k-steps, this wave's 256 dims
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
                for (int kp = 0; kp < 2; ++kp) {
                    const unsigned off = 128u * (unsigned)(nt >> 1);
                    const s16x4 lo = lds_tr4(sb + v_off[kp][0][nt & 1] + off);
                    const s16x4 hi = lds_tr4(sb + v_off[kp][1][nt & 1] + off);
                    const s16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                                      __builtin_bit_cast(bf16x8, pb[kp]), acc[nt], 0, 0, 0);
                }
            }
        }

        // end of segment: write this wave's 32 rows x 256 dims
        const int nsplit = sload(p.splits + cs.b + 1) - sload(p.splits + cs.b);
        const int slot = cs.b == b0 ? first_slot : sload(p.splits + cs.b);
        const float inv = lrun > 0.f ? 1.f / lrun : 0.f;
        if (nsplit == 1) {
            uint16_t* o = p.out + ((size_t)cs.b * p.rows_total + row) * kDv + 256 * kh + 4 * h;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    ushort4 v;
                    v.x = bf16_rne(acc[nt][4 * j + 0] * inv);
                    v.y = bf16_rne(acc[nt][4 * j + 1] * inv);
                    v.z = bf16_rne(acc[nt][4 * j + 2] * inv);
                    v.w = bf16_rne(acc[nt][4 * j + 3] * inv);
                    *(ushort4*)(o + 32 * nt + 8 * j) = v;
                }
        } else {
            float* o = p.part_o + ((size_t)slot * p.rows_total + row) * kDv + 256 * kh + 4 * h;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f32x4 v = {acc[nt][4 * j + 0] * inv, acc[nt][4 * j + 1] * inv,
                               acc[nt][4 * j + 2] * inv, acc[nt][4 * j + 3] * inv};
                    *(f32x4*)(o + 32 * nt + 8 * j) = v;
                }
        }
        if (kh == 0 && h == 0) {
            const float lse = lrun > 0.f ? (mrun + __log2f(lrun)) * kLn2 : -INFINITY;
            if (nsplit == 1) p.lse[(size_t)cs.b * p.rows_total + row] = lse;
            else p.part_lse[(size_t)slot * p.rows_total + row] = lse;
        }
        // (the next segment's query loads wait for these stores and every copy
        // in flight, so the copy counts of the next slot waits stay exact)
        cs = next_segment(p, cs.b + 1, b0, j0, b1, j1);
    }
}

// ---------------------------------------------------------------- split combine

// Merge split partials by their log-sum-exp: out = sum_k exp(lse_k - L) o_k,
// lse = L = log sum_k exp(lse_k). One thread per 4 dims of one (sequence, row);
// sequences with no block get out = 0, lse = -inf; unsplit ones were written by
// the decode kernel.
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p)
{
    constexpr int U = 8;                                    // partials in flight per thread
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
    float mx = -INFINITY;
    for (int k = 0; k < ns; k += U) {
        float w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = (k + u < ns) ? lse_col[(size_t)(k + u) * p.rows_total] : -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) mx = fmaxf(mx, w[u]);
    }
    if (ns == 0 || mx == -INFINITY) {
        *(ushort4*)o = make_ushort4(0, 0, 0, 0);
        if (t == 0) *lo = -INFINITY;
        return;
    }
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    const float* o_col = p.part_o + ((size_t)s0 * p.rows_total + row) * kDv + 4 * t;
    for (int k = 0; k < ns; k += U) {
        f32x4 v[U];
        float w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = k + u < ns;
            w[u] = ok ? lse_col[(size_t)(k + u) * p.rows_total] : -INFINITY;
            v[u] = ok ? *(const f32x4*)(o_col + (size_t)(k + u) * p.rows_total * kDv) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float e = __expf(w[u] - mx);
            wsum += e;
            a += v[u] * e;
        }
    }
    const float inv = 1.f / wsum;
    ushort4 r;
    r.x = bf16_rne(a[0] * inv);
    r.y = bf16_rne(a[1] * inv);
    r.z = bf16_rne(a[2] * inv);
    r.w = bf16_rne(a[3] * inv);
    *(ushort4*)o = r;
    if (t == 0) *lo = mx + __logf(wsum);
}

hipError_t launch_decode(const DecodeParams& p, int num_units, int head_groups, int rows_wg, hipStream_t stream)
{
    dim3 grid(num_units, head_groups);
    switch (rows_wg) {
    case 16: hipLaunchKernelGGL((decode_stream_kernel<1>), grid, dim3(256), 0, stream, p); break;
    case 64: hipLaunchKernelGGL(decode_wide_kernel, grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream)
{
    dim3 grid((p.rows_total + 1) / 2, p.batch);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mla
