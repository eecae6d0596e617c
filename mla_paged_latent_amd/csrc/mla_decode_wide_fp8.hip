// MLA decode over the FP8 latent cache, wide kernel (gfx950): 64 query rows
// per workgroup on v_mfma_f32_32x32x16_bf16, for s_q * h_q a multiple of 64.
//
// The method is the decode attention of the bf16 kernels (FlashMLA explainer,
// theflyingbirds.in, section 4.1.1; "OpenSourceWeek Day 1: FlashMLA",
// bibleofai.com, "How KV Caching Works?", "How MLA Optimizes Memory Usage?")
// over a cache stored in 8-bit floats with one float32 scale per row -- the
// FP8 support the explainer names under section 9, "Future Directions".
//
// The work split is the bf16 wide kernel's (four waves; wave w = kh + 2 th
// contracts cached columns [288 kh, +288) of token half th against both row
// groups; the partial score tiles are summed through LDS; the token halves
// exchange row maxima; wave w accumulates output dims [128 w, +128) of all 64
// rows). What changes is the operand path:
//  * a block is staged as two 32-token FP8 slots (the code rows laid out as
//    in the FP8 streaming kernel: 37-chunk rows), 38 KB instead of 72 KB, in
//    38 one-KB copies spread over the QK^T matrix ops, and its 64 row scales
//    go to a 256-byte area of their own in one 16-lane copy, so that every
//    code copy has the same form (a scalar base plus a lane offset held in
//    registers);
//  * K fragments are 8-byte reads of codes turned into bf16 exactly before
//    the matrix op; V^T fragments come from ds_read_b64_tr_b8 (in each 16-lane
//    group output lane j byte e is byte j % 8 of source lane 2 e + j / 8), one
//    read per 32 dims x 16 tokens, then the same conversion;
//  * the row scale multiplies the scores (S_t * scale_t) and P (P_t * scale_t
//    before PV); the row sums use the unscaled P. Scales of rows past the end
//    of a sequence may hold anything and are masked, never multiplied.
#include "mla_device.h"

namespace mla {

namespace {

constexpr int kF8BlockB = 2 * kF8SlotB;            // 38,912 B: one 64-token block
constexpr int kXBf = 4096;                          // LDS inbox of each wave
constexpr int kScaleB = 256;                        // the 64 row scales of a block
constexpr int kLdsF = 2 * kF8BlockB + 4 * kXBf + 2 * kScaleB;      // 94,720 B
constexpr unsigned kXMaxF = 0, kXPF = 128, kXSumF = 2176;

__device__ __forceinline__ float lds_ff(unsigned addr) { return *(const lds_f32*)(uintptr_t)addr; }

// Copy c (0..37) of a block's codes: slot c / 19, copy c % 19 of that slot.
// Lane map as in the FP8 streaming kernel: position pos of the slot holds
// chunk ch of slot row r (pp = pos minus the pad chunk before row 16, r = pp /
// 37 = (pp * 1772) >> 16 exactly for pp < 2367); pad chunks, positions past
// the last row and rows past the `valid` real rows of the block read the
// block's first row. Returns the lane's byte offset from the block's first
// code row.
__device__ __forceinline__ unsigned f8_copy_offset(int valid, int c, int lane)
{
    const int hb = c >= 19 ? 1 : 0;
    const int i = c - 19 * hb;
    const int pos = i * 64 + lane;
    const int pp = pos - (pos >= kF8Row16 ? 1 : 0);
    const int r = (int)(__umul24((unsigned)pp, 1772u) >> 16);
    const int ch = pp - kF8Chunks * r;
    const bool data = pos != kF8Row16 - 1 && ch < 36 && r < 32;
    int br = 32 * hb + r;
    br = br < valid ? br : 0;
    return data ? (unsigned)(br * kDqk + 16 * ch) : 0u;
}

// Issue code copy c of the block at cache row row0 with this lane's offset `off`.
__device__ __forceinline__ void f8_block_copy(const unsigned char* codes, size_t row0, unsigned off,
                                              unsigned dst_block, int c)
{
    const int hb = c >= 19 ? 1 : 0;
    const int i = c - 19 * hb;
    dma16s(codes + row0 * kDqk, off, dst_block + (unsigned)hb * kF8SlotB + (unsigned)i * 1024u);
}

}  // namespace

__global__ __launch_bounds__(256) void decode_wide_fp8_kernel(DecodeParams p)
{
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kLdsF];
    const unsigned lds0 = lds_base(smem);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kh = wave & 1;                                // column half; owned row group
    const int th = wave >> 1;                               // token half of the block for QK^T
    const int h = lane >> 5;
    const int r32 = lane & 31;
    const unsigned char* codes = (const unsigned char*)p.kcache;

    const i32x8 meta = sload8(p.meta + (size_t)blockIdx.x * kMetaInts);
    const int b0 = meta[0];
    const int j0 = meta[1];
    const int b1 = meta[2];
    const int j1 = meta[3];
    const int first_slot = meta[6];

    const int row0 = blockIdx.y * 64 + r32;                 // this lane's row in row group 0 (+32: group 1)
    const int iq_own = (row0 + 32 * kh) / p.h_q;            // new-token index of the owned row
    const float c = p.scale_log2;
    const unsigned xin = lds0 + 2 * kF8BlockB;              // inbox of wave 0
    const unsigned xmine = xin + (unsigned)wave * kXBf;
    const unsigned scl0 = xin + 4 * kXBf;                   // row scales of LDS block 0 (block 1: + kScaleB)

    // Block-table window of the copy cursor: lane i holds entry tw_j + i of
    // sequence tw_b (loaded speculatively for the unit's first block before
    // its segment is known). A window is loaded where the cursor leaves the
    // previous one and read (readlane) only at the next block's copies, after
    // the wait for the block in flight, so the load never stalls a wave.
    int tw_b = b0, tw_j = j0;
    int tabv = b0 < p.batch ? table_window(p, tw_b, tw_j, lane) : 0;
    Segment is = next_segment(p, b0, b0, j0, b1, j1);   // copy cursor
    if (is.b >= p.batch) return;
    int itok = is.tb;
    auto cover = [&]() {                                   // the window holds the cursor's block
        if (is.b != tw_b || (itok >> 6) - tw_j >= 64) {
            tw_b = is.b;
            tw_j = itok >> 6;
            tabv = table_window(p, tw_b, tw_j, lane);
        }
    };
    cover();
    Segment cs = is;                                       // compute cursor
    // first cache row of the block at the copy cursor
    auto copy_row0 = [&]() {
        return (size_t)safe_page(__builtin_amdgcn_readlane(tabv, (itok >> 6) - tw_j), p.nblocks) * kPage;
    };

    // this wave copies c = wave + 4k of each block's codes (10 copies for waves 0-1,
    // 9 for 2-3, whose last slot goes to the row scales: wave 2 copies them); the
    // lane offsets of a whole block are computed once and kept in registers
    unsigned coff[10];
#pragma unroll
    for (int k = 0; k < 10; ++k) coff[k] = f8_copy_offset(kPage, wave + 4 * k, lane);
    int n_issued = 0;
    // copy k of this wave for the block at the copy cursor (k == ncopy: wave 2's row scales)
    auto copy_one = [&](int k, unsigned off, size_t row0) {
        if (k < 9 || wave < 2) {
            f8_block_copy(codes, row0, off, lds0 + (unsigned)(n_issued & 1) * kF8BlockB, wave + 4 * k);
        } else if (wave == 2 && lane < 16) {
            dma16s((const unsigned char*)(p.kscale + row0), 16u * (unsigned)lane,
                   scl0 + (unsigned)(n_issued & 1) * kScaleB);
        }
    };
    auto copy_end = [&]() {
        ++n_issued;
        itok += kPage;
        if (itok >= is.te) {
            is = next_segment(p, is.b + 1, b0, j0, b1, j1);
            itok = is.tb;
        }
        if (is.b < p.batch) cover();
    };
    {
        const int valid = is.te - itok;
        const size_t crow = copy_row0();
        for (int k = 0; k < 10; ++k) copy_one(k, f8_copy_offset(valid, wave + 4 * k, lane), crow);
        copy_end();
    }

    // QK^T A operand: token row tokA of the slot, the lane's 8 codes of k-step ks
    // at chunk 18 kh + ks, byte 8 h
    const int tokA = token_of_row(r32);
    const unsigned k_base = f8_row(tokA) + 16u * (unsigned)(18 * kh) + 8u * (unsigned)h;
    // PV A operand (transposed V) via ds_read_b64_tr_b8: source lane s of 16-lane
    // group G reads token token_of_row(16 kp + 8 (e / 4) + 4 (G / 2) + e % 4), e = s / 2,
    // dims 128 wave + 32 dt + 16 (G % 2) + 8 (s % 2) .. + 8
    const int G = lane >> 4, sl = lane & 15, e8 = sl >> 1;
    unsigned v_base[2];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp)
        v_base[kp] = f8_row(token_of_row(16 * kp + 8 * (e8 >> 2) + 4 * (G >> 1) + (e8 & 3))) +
                     (unsigned)(128 * wave + 16 * (G & 1) + 8 * (sl & 1));
    // scale of element i of the owned S^T tile: token token_of_row(8 (i / 4) + 4 h + i % 4) of the slot
    int n = 0;                                              // block being computed
    while (cs.b < p.batch) {
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

        for (int t0 = cs.tb; t0 < cs.te; t0 += kPage, ++n) {
            // block n has landed and every wave is done with block n - 1
            MLA_WAIT_VM(0);
            wg_barrier();
            // the next block goes into the LDS block that block n - 1 left: its copies
            // are spread over the QK^T matrix ops below
            const bool more = is.b < p.batch;
            const bool whole = is.te - itok >= kPage;
            if (more && !whole) {                           // the end of a segment: copied here
                const int valid = is.te - itok;
                const size_t crow = copy_row0();
                for (int k = 0; k < 10; ++k) copy_one(k, f8_copy_offset(valid, wave + 4 * k, lane), crow);
            }
            const unsigned blk = lds0 + (unsigned)(n & 1) * kF8BlockB;
            const unsigned sb = blk + (unsigned)th * kF8SlotB;

            // ---- partial S^T over this wave's column half: s0 owned row group, s1 the other
            f32x16 s0, s1;
#pragma unroll
            for (int i = 0; i < 16; ++i) { s0[i] = 0.f; s1[i] = 0.f; }
            // (two copies of the loop, with and without the spread copies, so that no
            // branch sits between its matrix ops)
            auto qk = [&](auto with_copy) {
                size_t crow = 0;
                if constexpr (decltype(with_copy)::value) crow = copy_row0();
                u32x2 kv[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) kv[ks] = *(const __attribute__((address_space(3))) u32x2*)(uintptr_t)(sb + k_base + 16u * ks);
                // K fragments are converted one k-step ahead (ping-pong), under the previous matrix ops
                bf16x8 a2[2];
                a2[0] = e4m3x8_to_bf16(kv[0]);
#pragma unroll
                for (int ks = 0; ks < 18; ++ks) {
                    __builtin_amdgcn_sched_barrier(0);
                    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2[ks & 1], qf[0][ks], s0, 0, 0, 0);
                    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2[ks & 1], qf[1][ks], s1, 0, 0, 0);
                    if (ks + 1 < 18) a2[(ks + 1) & 1] = e4m3x8_to_bf16(kv[(ks + 1) & 3]);
                    if (ks + 4 < 18) kv[ks & 3] = *(const __attribute__((address_space(3))) u32x2*)(uintptr_t)(sb + k_base + 16u * (ks + 4));
                    if constexpr (decltype(with_copy)::value)
                        if (ks < 10) copy_one(ks, coff[ks], crow);
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            if (more && whole)
                qk(std::true_type{});
            else
                qk(std::false_type{});
            if (more) copy_end();
            // row scales of the owned tile's tokens (element i: token 32 th + token_of_row(8(i/4) + 4h + i%4)
            // of the block), read here so that their latency passes under the exchange barrier
            float scl[16];
            const unsigned sclb = scl0 + (unsigned)(n & 1) * kScaleB + 128u * (unsigned)th;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                scl[i] = lds_ff(sclb + 4u * (unsigned)token_of_row(8 * (i >> 2) + 4 * h + (i & 3)));
            // ---- score exchange: send the partner's row group (s1), add the partner's half of mine (s0)
            f32x16 s = s0;
            {
                const unsigned xp = xin + (unsigned)(wave ^ 1) * kXBf + 16u * lane;
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

            // ---- row scales, scale and mask the owned tile; element i is token
            // t0 + 32 th + token_of_row(8(i/4) + 4h + i%4) of row group kh
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int tr = token_of_row(8 * (i >> 2) + 4 * h + (i & 3));
                const bool vis = t0 + 32 * th + tr < lim;
                s[i] = vis ? s[i] * (scl[i] * c) : -INFINITY;
                scl[i] = vis ? scl[i] : 0.f;
            }
            {
                float m4[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) m4[j] = fmaxf(fmaxf(s[4 * j], s[4 * j + 1]), fmaxf(s[4 * j + 2], s[4 * j + 3]));
                const float tmax = xor32_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
                if (h == 0) *(lds_f32*)(uintptr_t)(xmine + kXMaxF + 4u * r32) = tmax;
            }
            wg_barrier();

            // ---- running max of all 64 rows (the same in every wave), lazy rescale
#pragma unroll
            for (int rg = 0; rg < 2; ++rg) {
                const float mb = fmaxf(lds_ff(xin + (unsigned)rg * kXBf + kXMaxF + 4u * r32),
                                       lds_ff(xin + (unsigned)(rg + 2) * kXBf + kXMaxF + 4u * r32));
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
            // ---- P of the owned tile: row sums of P, P * scale posted as bf16 P^T operands
            {
                const float mk = kh ? mrun[1] : mrun[0];
                const float muse = mk == -INFINITY ? 0.f : mk;
                float pv[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) pv[i] = __builtin_amdgcn_exp2f(s[i] - muse);
                float q4[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) q4[j] = (pv[4 * j] + pv[4 * j + 1]) + (pv[4 * j + 2] + pv[4 * j + 3]);
                lrun += xor32_sum((q4[0] + q4[1]) + (q4[2] + q4[3]));
#pragma unroll
                for (int kp = 0; kp < 2; ++kp) {
                    u32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[e] = pack_bf16x2(pv[8 * kp + 2 * e] * scl[8 * kp + 2 * e], pv[8 * kp + 2 * e + 1] * scl[8 * kp + 2 * e + 1]);
                    *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(xmine + kXPF + 1024u * kp + 16u * lane) = w;
                }
            }
            wg_barrier();

            // ---- O^T += V^T (P scale)^T: this wave's 128 dims, both row groups, both token halves
#pragma unroll
            for (int tq = 0; tq < 2; ++tq) {
                const unsigned vb = blk + (unsigned)tq * kF8SlotB;
                bf16x8 pf[2][2];
#pragma unroll
                for (int rg = 0; rg < 2; ++rg)
#pragma unroll
                    for (int kp = 0; kp < 2; ++kp)
                        pf[rg][kp] = __builtin_bit_cast(bf16x8, lds_load16(xin + (unsigned)(rg + 2 * tq) * kXBf + kXPF +
                                                                           1024u * kp + 16u * lane));
                auto load_v = [&](int k) {
                    const int dt = k >> 1, kp = k & 1;
                    const auto t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) i32x2*)(uintptr_t)(vb + v_base[kp] + 32u * (unsigned)dt));
                    return u32x2{(unsigned)t[0], (unsigned)t[1]};
                };
                u32x2 va[2];
                va[0] = load_v(0);
                va[1] = load_v(1);
                bf16x8 a2[2];
                a2[0] = e4m3x8_to_bf16(va[0]);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    __builtin_amdgcn_sched_barrier(0);
                    const int dt = k >> 1, kp = k & 1;
                    acc[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2[k & 1], pf[0][kp], acc[0][dt], 0, 0, 0);
                    acc[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2[k & 1], pf[1][kp], acc[1][dt], 0, 0, 0);
                    if (k + 1 < 8) a2[(k + 1) & 1] = e4m3x8_to_bf16(va[(k + 1) & 1]);
                    if (k + 2 < 8) va[k & 1] = load_v(k + 2);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- end of segment: row sums of both token halves, then this wave's 128 dims of 64 rows
        if (h == 0) *(lds_f32*)(uintptr_t)(xmine + kXSumF + 4u * r32) = lrun;
        wg_barrier();
        const int nsplit = sp1 - sp0;
        const int slot = cs.b == b0 ? first_slot : sp0;
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
            const float lt = lds_ff(xin + (unsigned)rg * kXBf + kXSumF + 4u * r32) +
                             lds_ff(xin + (unsigned)(rg + 2) * kXBf + kXSumF + 4u * r32);
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            const int row = row0 + 32 * rg;
            if (nsplit == 1) {
                uint16_t* o = p.out + ((size_t)cs.b * p.rows_total + row) * kDv + 128 * wave + 4 * h;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        u32x2 v;
                        v[0] = pack_bf16x2(acc[rg][dt][4 * j + 0] * inv, acc[rg][dt][4 * j + 1] * inv);
                        v[1] = pack_bf16x2(acc[rg][dt][4 * j + 2] * inv, acc[rg][dt][4 * j + 3] * inv);
                        *(u32x2*)(o + 32 * dt + 8 * j) = v;
                    }
            } else {
                float* o = p.part_o + ((size_t)slot * p.rows_total + row) * kDv + 128 * wave + 4 * h;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        f32x4 v = {acc[rg][dt][4 * j + 0] * inv, acc[rg][dt][4 * j + 1] * inv,
                                   acc[rg][dt][4 * j + 2] * inv, acc[rg][dt][4 * j + 3] * inv};
                        *(f32x4*)(o + 32 * dt + 8 * j) = v;
                    }
            }
            if (wave == rg && h == 0) {
                const float lse = lt > 0.f ? (mrun[rg] + __log2f(lt)) * kLn2 : -INFINITY;
                if (nsplit == 1) p.lse[(size_t)cs.b * p.rows_total + row] = lse;
                else p.part_lse[(size_t)slot * p.rows_total + row] = lse;
            }
        }
        cs = next_segment(p, cs.b + 1, b0, j0, b1, j1);
    }
}

hipError_t launch_wide_fp8(const DecodeParams& p, dim3 grid, hipStream_t stream)
{
    hipLaunchKernelGGL(decode_wide_fp8_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mla
