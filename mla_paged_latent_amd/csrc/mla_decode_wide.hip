// MLA decode, wide kernel (gfx950): 64 query rows per workgroup on
// v_mfma_f32_32x32x16_bf16. Built with the VGPR form of the matrix ops so the
// output accumulators live in VGPRs, where the online-softmax rescale can
// scale them in place (AGPR accumulators would need a copy through VGPRs).
#include "mla_device.h"

namespace mla {

// ---------------------------------------------------------------- wide kernel
//
// 64 query rows (two row groups of 32) per workgroup, four waves, one 64-token
// cache block per step, two blocks of LDS (the one being computed and the
// next one in flight). Every cached byte the workgroup uses is read from LDS
// once:
//  * QK^T: wave w = kh + 2 th contracts cached columns [288 kh, 288 kh + 288)
//    of token half th (tokens [32 th, 32 th + 32) of the block) against both
//    row groups (its half of Q for all 64 rows sits in AGPRs); each K fragment
//    feeds two matrix ops. The partial S^T tiles of the two column halves are
//    summed through LDS: afterwards wave (kh, th) holds the scores of row
//    group kh on token half th.
//  * Softmax: the two token halves' row maxima are exchanged, so every wave
//    knows the running max of all 64 rows (the same for every wave) and the
//    exponentials P of its own tile, which it posts to LDS.
//  * PV: wave w accumulates output dims [128 w, 128 w + 128) of all 64 rows
//    over the whole block (each V^T fragment feeds two matrix ops, one per
//    row group), reading the four P^T tiles back from LDS.
// S^T = K Q^T puts the scores in the layout of the P^T operand of
// O^T = V^T P^T, so P is packed to bf16 where it is computed. Block halves
// hold rows of 1152 B with their chunks permuted (swz below), which with the
// token permutation keeps b128 and transpose reads conflict free.

constexpr int kHalfB = 32 * kRowBytes;          // 36,864 B: 32 token rows, 36 copies of 1 KB
constexpr int kBlockB = 2 * kHalfB;             // 73,728 B: one cache block
constexpr int kXB = 4096;                       // LDS inbox of each wave
constexpr int kLdsB = 2 * kBlockB + 4 * kXB;    // 163,840 B
// An inbox holds the partner's partial S^T tile during the score exchange
// (all 4 KB), afterwards its owner's row maxima, P^T tile and row sums.
constexpr unsigned kXMax = 0, kXP = 128, kXSum = 2176;

// Result rows.
//
// A lane of a 32x32 matrix-op output tile holds 16 dims of one row, so stores
// straight from the accumulators would write 32 rows x 16 or 32 B per
// instruction. The rows are staged row-major in LDS instead (one 16-byte pad
// chunk per row spreads the lanes' writes of an instruction over the banks),
// after which each store instruction writes 1 KB of one row.
constexpr unsigned kStgB16 = 2 * kDv + 16;          // a staged bf16 row
constexpr unsigned kStgF32 = 4 * kDv + 16;          // a staged fp32 row
constexpr unsigned kStgBytes = 64 * kStgB16;        // 64 bf16 rows, or 32 fp32 rows
static_assert(32 * kStgF32 <= kStgBytes, "fp32 staging fits");
static_assert(kStgBytes <= kBlockB, "result staging fits a block buffer");

// The 64 rows of a workgroup (rows_out: their first row in out, or in the split
// partials when !final), acc[rg][dt][4 j + e] = dim 128 wave + 32 dt + 8 j + 4 h + e
// of row 32 rg + r32, scaled by inv[rg]. stg: kStgBytes of LDS that no other
// wave uses until the next workgroup barrier after this call.
__device__ __forceinline__ void store_rows_staged(const f32x16 (&acc)[2][4], const float (&inv)[2], unsigned stg,
                                                  int wave, int lane, bool final, uint16_t* rows_out,
                                                  float* rows_part)
{
    const int h = lane >> 5, r32 = lane & 31;
    if (final) {
        // bf16 rows; wave w then stores rows 16 w .. 16 w + 15
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    u32x2 v;
                    v[0] = pack_bf16x2(acc[rg][dt][4 * j + 0] * inv[rg], acc[rg][dt][4 * j + 1] * inv[rg]);
                    v[1] = pack_bf16x2(acc[rg][dt][4 * j + 2] * inv[rg], acc[rg][dt][4 * j + 3] * inv[rg]);
                    *(__attribute__((address_space(3))) u32x2*)(uintptr_t)(
                        stg + (unsigned)(32 * rg + r32) * kStgB16 + 2u * (unsigned)(128 * wave + 32 * dt + 8 * j + 4 * h)) = v;
                }
        wg_barrier();
        uint16_t* o = rows_out + 8 * lane;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 16 * wave + i;
            *(s16x8*)(o + (size_t)r * kDv) = lds_load16(stg + (unsigned)r * kStgB16 + 16u * lane);
        }
    } else {
        // fp32 rows, one row group at a time; wave w stores rows 8 w .. 8 w + 7 of it
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
            if (rg) wg_barrier();                           // every wave has stored the first group
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 v = {acc[rg][dt][4 * j + 0] * inv[rg], acc[rg][dt][4 * j + 1] * inv[rg],
                                     acc[rg][dt][4 * j + 2] * inv[rg], acc[rg][dt][4 * j + 3] * inv[rg]};
                    *(lds_f32x4*)(uintptr_t)(stg + (unsigned)r32 * kStgF32 +
                                             4u * (unsigned)(128 * wave + 32 * dt + 8 * j + 4 * h)) = v;
                }
            wg_barrier();
            float* o = rows_part + (size_t)(32 * rg) * kDv + 4 * lane;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * wave + i;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    *(f32x4*)(o + (size_t)r * kDv + 256 * hf) =
                        *(const lds_f32x4*)(uintptr_t)(stg + (unsigned)r * kStgF32 + 1024u * hf + 16u * lane);
            }
        }
    }
}

// Maximum for the row maxima: scores are finite or -inf here (masked tokens are
// -inf, rows past a sequence's end hold finite copies), so the NaN-propagating
// IEEE maximum (v_maximum3_f32) gives fmaxf's result without the NaN-quieting
// operations fmaxf needs on values the compiler cannot prove canonical.
__device__ __forceinline__ float fmaxr(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float xor32_maxr(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxr(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lds_f(unsigned addr) { return *(const lds_f32*)(uintptr_t)addr; }

__global__ __launch_bounds__(256) void decode_wide_kernel(DecodeParams p)
{
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kLdsB];
    const unsigned lds0 = lds_base(smem);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kh = wave & 1;                                // column half; owned row group
    const int th = wave >> 1;                               // token half of the block for QK^T
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

    const int row0 = blockIdx.y * 64 + r32;                 // this lane's row in row group 0 (+32: group 1)
    const int iq_own = (row0 + 32 * kh) / p.h_q;            // new-token index of the owned row
    const float c = p.scale_log2;
    const unsigned xin = lds0 + 2 * kBlockB;                // inbox of wave 0
    const unsigned xmine = xin + (unsigned)wave * kXB;

    // Block-table window of the copy cursor: lane i holds entry tw_j + i of
    // sequence tw_b (loaded speculatively for the unit's first block before
    // its segment is known). A window is loaded where the cursor leaves the
    // previous one and read (readlane) only at the next block's copies, after
    // the wait for the block in flight, so the load never stalls a wave.
    int tw_b = b0, tw_j = j0;
    int tabv = b0 < p.batch ? table_window(p, tw_b, tw_j, lane) : 0;
    Segment is = next_segment(p, b0, b0, j0, b1, j1);      // copy cursor
    if (is.b >= p.batch) return;
    int itok = is.tb;
    auto cover = [&]() {                                    // the window holds the cursor's block
        if (is.b != tw_b || (itok >> 6) - tw_j >= 64) {
            tw_b = is.b;
            tw_j = itok >> 6;
            tabv = table_window(p, tw_b, tw_j, lane);
        }
    };
    cover();
    Segment cs = is;                                        // compute cursor

    // This wave's copies of a block: copy i = wave + 4k of each half (36 per
    // half); lane l of copy i reads chunk c of row r (72 r + c = 64 i + l) of
    // the half and lands at its permuted position swz(r, c).
    unsigned goff[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const int q = (wave + 4 * k) * 64 + lane;
        const int r = q / kChunks;
        goff[k] = swz(r, q - r * kChunks);
    }
    int n_issued = 0;
    // The next block of the copy cursor goes to LDS block (n_issued % 2):
    // copy_src / copy_dst give the global page and this wave's LDS base.
    auto copy_src = [&]() {
        const int page = safe_page(__builtin_amdgcn_readlane(tabv, (itok >> 6) - tw_j), p.nblocks);
        return (const unsigned char*)p.kcache + (size_t)page * kPageBytes;
    };
    auto copy_dst = [&]() { return lds0 + (unsigned)(n_issued & 1) * kBlockB + (unsigned)wave * 1024u; };
    // copy k (0..17) of a whole block: half k / 9, copy k % 9 of that half
    auto copy_full = [&](const unsigned char* gbase, unsigned dst, int k) {
        const unsigned hb = k < 9 ? 0u : (unsigned)kHalfB;
        dma16s(gbase, goff[k % 9] + hb, dst + hb + 4096u * (unsigned)(k % 9));
    };
    // advance the copy cursor past the block just copied
    auto copy_end = [&]() {
        ++n_issued;
        itok += kPage;
        if (itok >= is.te) {
            is = next_segment(p, is.b + 1, b0, j0, b1, j1);
            itok = is.tb;
        }
        if (is.b < p.batch) cover();
    };
    // Copy the next block all at once. Rows past the segment's end are copied
    // from the block's first row (finite data, masked to p = 0).
    auto issue = [&]() {
        const unsigned char* gbase = copy_src();
        const unsigned dst = copy_dst();
        const int valid = is.te - itok;
        if (valid >= kPage) {
#pragma unroll
            for (int k = 0; k < 18; ++k) copy_full(gbase, dst, k);
        } else {
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int k = 0; k < 9; ++k) {
                    const int r = (int)(goff[k] / kRowBytes);
                    const unsigned col = goff[k] - (unsigned)(r * kRowBytes);
                    const int br = 32 * hb + r;             // row of the block
                    const unsigned src = br < valid ? (unsigned)(br * kRowBytes) + col : col;
                    dma16s(gbase, src, dst + (unsigned)(hb * kHalfB) + 4096u * k);
                }
        }
        copy_end();
    };
    issue();

    // QK^T A operand (K rows): token row tokA; for k-step ks its chunk is
    // 36 kh + 2 ks + h (64 or more only for kh = 1, ks >= 14)
    const int tokA = token_of_row(r32);
    const unsigned k_row = (unsigned)(tokA * kRowBytes);
    const int k_f = swz_f(tokA);
    auto k_off = [&](int ks) {
        const int c = 36 * kh + 2 * ks + h;
        return k_row + (unsigned)(((kh && ks >= 14) ? (c ^ (k_f & 7)) : (c ^ k_f)) << 4);
    };
    // PV A operand (transposed V): source row token_of_row(16 kp + 8 half + 4h + i16/4),
    // dims 128 wave + 32 dt + 16 dh + 4 (i16 % 4), i.e. chunk 16 wave + 4 dt + 2 dh + (i16 % 4)/2 (< 64)
    unsigned v_row[2][2];
    int v_f[2][2];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int r = token_of_row(16 * kp + 8 * half + 4 * h + (i16 >> 2));
            v_row[kp][half] = (unsigned)(r * kRowBytes) + 8u * (unsigned)(i16 & 1);
            v_f[kp][half] = swz_f(r);
        }
    const int v_c = 16 * wave + 2 * dh + ((i16 & 3) >> 1);

    int n = 0;                                              // block being computed
    while (cs.b < p.batch) {
        // new segment: this wave's column half of Q for both row groups (qf[0]:
        // the owned group kh, qf[1]: the other), fresh softmax state
        const int sp0 = cload(p.splits + cs.b), sp1 = cload(p.splits + cs.b + 1);
        bf16x8 qf[2][18];
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
            const uint16_t* qrow = p.q + ((size_t)cs.b * p.rows_total + row0 + 32 * (rg ^ kh)) * kDqk + 288 * kh + 8 * h;
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) qf[rg][ks] = __builtin_bit_cast(bf16x8, *(const s16x8*)(qrow + 16 * ks));
        }
        settle_loads();
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) asm volatile("" : "+a"(qf[rg][ks]));
        // (the split counts are needed only at the segment's end; taking them
        // here, after the query loads, keeps the block loop free of pending
        // scalar loads, which would make its LDS waits wait for everything)
        asm volatile("" : : "s"(sp0), "s"(sp1));
        f32x16 acc[2][4];
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[rg][dt][i] = 0.f;
        float mrun[2] = {-INFINITY, -INFINITY};
        float lrun = 0.f;                                   // owned rows, this wave's token half
        const int lim = min(cs.te, p.causal ? cs.L - (p.s_q - 1 - iq_own) : cs.L);
        // lane 0 holds the wave's first owned row, whose visible prefix is the shortest
        const int lim_lo = __builtin_amdgcn_readfirstlane(lim);

        for (int t0 = cs.tb; t0 < cs.te; t0 += kPage, ++n) {
            // block n has landed and every wave is done with block n - 1: its
            // LDS block takes the next copy
            MLA_WAIT_VM(0);
            wg_barrier();
            // The next block (into the LDS block that block n - 1 just left):
            // a whole one is copied during the QK^T below, one copy per pair of
            // matrix ops, so that the waits of the copy issue overlap the matrix
            // work; a partial one (the end of a segment) is copied here.
            const bool spread = is.b < p.batch && is.te - itok >= kPage;
            if (is.b < p.batch && !spread) issue();
            const unsigned blk = lds0 + (unsigned)(n & 1) * kBlockB;

            // ---- partial S^T over this wave's column half: s0 owned row group, s1 the other
            f32x16 s0, s1;
#pragma unroll
            for (int i = 0; i < 16; ++i) { s0[i] = 0.f; s1[i] = 0.f; }
            auto qk = [&](auto with_copy) {
                const unsigned sb = blk + (unsigned)th * kHalfB;
                const unsigned char* gbase = copy_src();
                const unsigned dst = copy_dst();
                s16x8 kv[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) kv[ks] = lds_load16(sb + k_off(ks));
#pragma unroll
                for (int ks = 0; ks < 18; ++ks) {
                    __builtin_amdgcn_sched_barrier(0);
                    const bf16x8 a = __builtin_bit_cast(bf16x8, kv[ks & 3]);
                    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[0][ks], s0, 0, 0, 0);
                    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[1][ks], s1, 0, 0, 0);
                    if (ks + 4 < 18) kv[ks & 3] = lds_load16(sb + k_off(ks + 4));
                    if constexpr (decltype(with_copy)::value) copy_full(gbase, dst, ks);
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            if (spread) {
                qk(std::true_type{});
                copy_end();
            } else {
                qk(std::false_type{});
            }
            // ---- score exchange: send the partner's row group (s1), add the partner's half of mine (s0)
            f32x16 s = s0;
            {
                const unsigned xp = xin + (unsigned)(wave ^ 1) * kXB + 16u * lane;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *(lds_f32x4*)(uintptr_t)(xp + 1024 * j) = f32x4{s1[4 * j], s1[4 * j + 1], s1[4 * j + 2], s1[4 * j + 3]};
            }
            wg_barrier();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 o = *(const lds_f32x4*)(uintptr_t)(xmine + 16u * lane + 1024 * j);
                s[4 * j] += o[0]; s[4 * j + 1] += o[1]; s[4 * j + 2] += o[2]; s[4 * j + 3] += o[3];
            }

            // ---- scale and mask the owned tile; element i is token
            // t0 + 32 th + token_of_row(8(i/4) + 4h + i%4) of row group kh.
            // Unmasked (and with a positive scale) s keeps the raw scores and
            // cs is the scale; masked, s holds scaled scores and cs = 1.
            float cs_ = c;
            if (!(t0 + kPage <= lim_lo && c > 0.f)) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int t = t0 + 32 * th + token_of_row(8 * (i >> 2) + 4 * h + (i & 3));
                    s[i] = (t < lim) ? s[i] * c : -INFINITY;
                }
                cs_ = 1.f;
            }
            {
                float m4[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) m4[j] = fmaxr(fmaxr(s[4 * j], s[4 * j + 1]), fmaxr(s[4 * j + 2], s[4 * j + 3]));
                const float tmax = xor32_maxr(fmaxr(fmaxr(m4[0], m4[1]), fmaxr(m4[2], m4[3])) * cs_);
                // (the inbox's score tile has been read: this wave's LDS ops run in order)
                if (h == 0) *(lds_f32*)(uintptr_t)(xmine + kXMax + 4u * r32) = tmax;
            }
            wg_barrier();

            // ---- running max of all 64 rows (the same in every wave), lazy rescale
#pragma unroll
            for (int rg = 0; rg < 2; ++rg) {
                const float mb = fmaxr(lds_f(xin + (unsigned)rg * kXB + kXMax + 4u * r32),
                                       lds_f(xin + (unsigned)(rg + 2) * kXB + kXMax + 4u * r32));
                const bool need = mb > mrun[rg] + kLazyTau;
                if (wave_any(need)) {
                    const float mnew = need ? mb : mrun[rg];
                    const float alpha = need ? __builtin_amdgcn_exp2f(mrun[rg] - mnew) : 1.f;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) acc[rg][dt] *= alpha;
                    if (rg == kh) lrun *= alpha;
                    mrun[rg] = mnew;
                }
            }
            // ---- P of the owned tile: row sums, bf16 P^T operands posted to LDS
            {
                const float mk = kh ? mrun[1] : mrun[0];
                const float muse = mk == -INFINITY ? 0.f : mk;
                float pv[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(s[i], cs_, -muse));
                float q4[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) q4[j] = (pv[4 * j] + pv[4 * j + 1]) + (pv[4 * j + 2] + pv[4 * j + 3]);
                lrun += xor32_sum((q4[0] + q4[1]) + (q4[2] + q4[3]));
#pragma unroll
                for (int kp = 0; kp < 2; ++kp) {
                    u32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(pv[8 * kp + 2 * e], pv[8 * kp + 2 * e + 1]);
                    *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(xmine + kXP + 1024u * kp + 16u * lane) = w;
                }
            }
            wg_barrier();

            // ---- O^T += V^T P^T: this wave's 128 dims, both row groups, both token halves
#pragma unroll
            for (int tq = 0; tq < 2; ++tq) {
                const unsigned sb = blk + (unsigned)tq * kHalfB;
                bf16x8 pf[2][2];
#pragma unroll
                for (int rg = 0; rg < 2; ++rg)
#pragma unroll
                    for (int kp = 0; kp < 2; ++kp)
                        pf[rg][kp] = __builtin_bit_cast(bf16x8, lds_load16(xin + (unsigned)(rg + 2 * tq) * kXB + kXP +
                                                                           1024u * kp + 16u * lane));
                s16x4 va[2][2];
                auto load_v = [&](int k, s16x4* d) {
                    const int dt = k >> 1, kp = k & 1;
                    const int c = v_c + 4 * dt;
                    d[0] = lds_tr4(sb + v_row[kp][0] + (unsigned)((c ^ v_f[kp][0]) << 4));
                    d[1] = lds_tr4(sb + v_row[kp][1] + (unsigned)((c ^ v_f[kp][1]) << 4));
                };
#pragma unroll
                for (int k = 0; k < 2; ++k) load_v(k, va[k]);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    __builtin_amdgcn_sched_barrier(0);
                    const int dt = k >> 1, kp = k & 1;
                    const s16x4 lo = va[k & 1][0], hi = va[k & 1][1];
                    const bf16x8 a = __builtin_bit_cast(bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
                    acc[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[0][kp], acc[0][dt], 0, 0, 0);
                    acc[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[1][kp], acc[1][dt], 0, 0, 0);
                    if (k + 2 < 8) load_v(k + 2, va[k & 1]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- end of segment: row sums of both token halves, then the 64 result
        // rows, staged in the LDS buffer of the segment's last block (free now:
        // every wave is past its PV, and the block in flight goes to the other
        // buffer).
        if (h == 0) *(lds_f32*)(uintptr_t)(xmine + kXSum + 4u * r32) = lrun;
        wg_barrier();
        const int nsplit = sp1 - sp0;
        const int slot = cs.b == b0 ? first_slot : sp0;
        const unsigned stg = lds0 + (unsigned)((n - 1) & 1) * kBlockB;
        float inv[2];
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
            const float lt = lds_f(xin + (unsigned)rg * kXB + kXSum + 4u * r32) +
                             lds_f(xin + (unsigned)(rg + 2) * kXB + kXSum + 4u * r32);
            inv[rg] = lt > 0.f ? 1.f / lt : 0.f;
            if (wave == rg && h == 0) {
                const int row = row0 + 32 * rg;
                const float lse = lt > 0.f ? (mrun[rg] + __log2f(lt)) * kLn2 : -INFINITY;
                if (nsplit == 1) p.lse[(size_t)cs.b * p.rows_total + row] = lse;
                else p.part_lse[(size_t)slot * p.rows_total + row] = lse;
            }
        }
        const size_t row_wg = (size_t)blockIdx.y * 64;      // the workgroup's first row
        store_rows_staged(acc, inv, stg, wave, lane, nsplit == 1, p.out + ((size_t)cs.b * p.rows_total + row_wg) * kDv,
                          p.part_o + ((size_t)slot * p.rows_total + row_wg) * kDv);
        // (the next block's barrier keeps the row sums and the staged rows until all read them)
        cs = next_segment(p, cs.b + 1, b0, j0, b1, j1);
    }
}

hipError_t launch_wide(const DecodeParams& p, dim3 grid, hipStream_t stream)
{
    hipLaunchKernelGGL(decode_wide_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mla
