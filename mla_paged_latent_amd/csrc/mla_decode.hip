// MLA decode kernel for gfx950 (CDNA4): paged latent cache -> LDS -> bf16 MFMA.
//
// What one workgroup does (unit u of the split-KV plan, head group hg):
//   for each segment (sequence b, blocks [j0, j1)) of its unit:
//     load its 16*NR query rows into VGPRs (MFMA B-operand layout);
//     for each cache block (64 tokens x 576 bf16 = 73,728 contiguous bytes):
//       copy the block into one of two LDS buffers with direct global->LDS
//       loads (the next block is in flight while this one is used), zeroing
//       rows past the sequence end so that they contribute exactly 0;
//       S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K rows from LDS);
//       scale, causal/length mask, online softmax in fp32 (exp2 domain);
//       O^T += V^T P^T on MFMA, V = first 512 columns of the same LDS rows,
//       P taken straight from the S^T accumulators (no LDS round trip);
//     merge the NK waves that split the tokens, then write out/lse, or a
//     normalised fp32 partial and its lse when the sequence is split.
//
// The method: decode-time attention of new queries over cached rows
// ("OpenSourceWeek Day 1: FlashMLA", bibleofai.com, "How KV Caching Works?")
// with one latent row shared by all heads (same page, "How MLA Optimizes
// Memory Usage?"), scaled dot-product softmax (FlashMLA explainer,
// theflyingbirds.in, section 4.1.1), 64-token pages (same explainer, 4.3.2),
// blocks staged on chip before use and read with contiguous accesses
// (explainer 4.2.1-4.2.2), softmax fused with the matrix products (4.2.3).
//
// Wave roles: NR row groups x NK token slices. Wave (rg, kk) owns query rows
// [16 rg, 16 rg + 16) of the workgroup and tokens [kk*64/NK, (kk+1)*64/NK) of
// every block; each wave keeps its own running max/sum/O and the NK slices are
// merged once per segment.
//
// Register layouts (v_mfma_f32_16x16x32_bf16: lane l, group g = l/16):
//   A operand: row (l%16), k = 8g..8g+7; B operand: column (l%16), same k;
//   D: column (l%16), rows 4g..4g+3.
//   S^T tile (tokens x rows): lane holds row (l%16), tokens 4g..4g+3 of a
//   16-token sub-tile -- exactly the P^T B-operand of the PV product when the
//   k index of element e is token 4g+e (sub-tile st0) or 4g+e-4 (st1).
//   O^T (512 dims x 16 rows): 32 tiles, lane holds row (l%16), dims 16nt+4g+i.
//
// LDS block layout: row r (token) is 72 chunks of 16 B followed by one unused
// 16 B pad, so the row stride is 1168 B: 8 consecutive rows reading the same
// chunk land on 8 different 16-byte bank groups, and every operand address is
// one per-lane base plus a compile-time offset.
#include "mla_common.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunks = kRowBytes / 16;          // 72 chunks of 16 B per row
constexpr int kSlots = kChunks + 1;              // 73 LDS slots per row (one pad)
constexpr int kLdsRow = kSlots * 16;             // 1168 B
constexpr int kDmaInstr = (kPage * kSlots + 63) / 64;   // 73 wave-wide 1 KB loads per block
constexpr int kBufBytes = kDmaInstr * 1024;      // 74,752 B
constexpr int kLdsBytes = 2 * kBufBytes;         // 149,504 B
constexpr int kObufStride = kDv + 4;             // fp32 row stride of the merge buffer

typedef __attribute__((address_space(3))) void lds_void;


__device__ __forceinline__ unsigned short bf16_bits_rne(float f)
{
    unsigned u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (unsigned short)(u >> 16);
}

// Issue the direct-to-LDS copy of one cache block. Rows >= valid are not read.
// Wave w issues 1 KB loads w, w+NW, ...; lane l of load i fills LDS bytes
// [1024 i + 16 l, +16), which is slot s of row r with 73 r + s = 64 i + l
// (slot 72 is the pad and is not loaded).
template <int NW>
__device__ __forceinline__ void issue_block(unsigned char* buf, const unsigned char* src, int valid, int wave, int lane)
{
#pragma unroll 1
    for (int i = wave; i < kDmaInstr; i += NW) {
        const int q = i * 64 + lane;
        const int r = q / kSlots;
        const int s = q - r * kSlots;
        if (r < valid && s < kChunks) {
            __builtin_amdgcn_global_load_lds((const void*)(src + r * kRowBytes + s * 16),
                                             (lds_void*)(buf + i * 1024), 16, 0, 0);
        }
    }
}

template <int NT>
__device__ __forceinline__ void zero_rows(unsigned char* buf, int first_row)
{
    const int n = (kPage - first_row) * kChunks;
    for (int k = threadIdx.x; k < n; k += NT) {
        const int r = first_row + k / kChunks;
        const int s = k % kChunks;
        *(uint4*)(buf + r * kLdsRow + s * 16) = make_uint4(0, 0, 0, 0);
    }
}

template <int NR, int NK>
__global__ __launch_bounds__(64 * NR * NK) void decode_kernel(DecodeParams p)
{
    constexpr int NW = NR * NK;
    constexpr int NT = 64 * NW;
    constexpr int MW = 16 * NR;          // query rows per workgroup
    constexpr int TW = kPage / NK;       // tokens per wave per block
    constexpr int NST = TW / 16;         // 16-token sub-tiles per wave per block
    static_assert(NST >= 1, "token slice too small");

    __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int rg = wave % NR;
    const int kk = wave / NR;
    const int g = lane >> 4;
    const int c16 = lane & 15;

    const int32_t* meta = p.meta + (size_t)blockIdx.x * kMetaInts;
    const int b_end = meta[2];
    const int j_end = meta[3];
    int b = meta[0];
    int jb = meta[1];
    int split = meta[4];

    const int row_wave = blockIdx.y * MW + rg * 16;      // first row of this wave's tile
    const int myrow = row_wave + c16;                    // the row this lane's stats belong to
    const int iq = myrow / p.h_q;                        // new-token index of that row

    for (; b <= b_end && b < p.batch; ++b, jb = 0, split = 0) {
        const int L = p.seqlens[b];
        const int nb = blocks_of(L);
        const int je = (b == b_end) ? j_end : nb;
        if (jb >= je) continue;
        const int lim = p.causal ? L - (p.s_q - 1 - iq) : L;   // tokens t < lim are visible to myrow
        const int32_t* table = p.block_table + (size_t)b * p.max_blocks;

        // queries: lane holds row myrow, columns 8g + 32ks .. +8
        bf16x8 qf[18];
        {
            const uint16_t* qrow = p.q + ((size_t)b * p.rows_total + myrow) * kDqk + 8 * g;
#pragma unroll
            for (int ks = 0; ks < 18; ++ks)
                qf[ks] = __builtin_bit_cast(bf16x8, *(const s16x8*)(qrow + 32 * ks));
        }
        float mrow = -INFINITY;
        float lrow = 0.f;
        f32x4 acc[32];
#pragma unroll
        for (int nt = 0; nt < 32; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

        {
            const unsigned char* src = (const unsigned char*)p.kcache + (size_t)table[jb] * kPageBytes;
            issue_block<NW>(smem, src, min(kPage, L - jb * kPage), wave, lane);
        }
        for (int j = jb; j < je; ++j) {
            unsigned char* buf = smem + ((j - jb) & 1) * kBufBytes;
            const int valid = min(kPage, L - j * kPage);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            if (valid < kPage) zero_rows<NT>(buf, valid);
            __syncthreads();
            if (j + 1 < je) {
                const unsigned char* src = (const unsigned char*)p.kcache + (size_t)table[j + 1] * kPageBytes;
                issue_block<NW>(smem + ((j + 1 - jb) & 1) * kBufBytes, src,
                                min(kPage, L - (j + 1) * kPage), wave, lane);
            }

            // ---- S^T = K Q^T over this wave's tokens
            const int tok0 = kk * TW;
            f32x4 s[NST];
#pragma unroll
            for (int st = 0; st < NST; ++st) {
                s[st] = f32x4{0.f, 0.f, 0.f, 0.f};
                const int r = tok0 + 16 * st + c16;
#pragma unroll
                for (int ks = 0; ks < 18; ++ks) {
                    const s16x8 a = *(const s16x8*)(buf + r * kLdsRow + (g + 4 * ks) * 16);
                    s[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), qf[ks], s[st], 0, 0, 0);
                    if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);
                }
            }

            // ---- scale, mask, online softmax (log2 domain)
            float tmax = -INFINITY;
#pragma unroll
            for (int st = 0; st < NST; ++st) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = j * kPage + tok0 + 16 * st + 4 * g + i;
                    const float v = (t < lim) ? s[st][i] * p.scale_log2 : -INFINITY;
                    s[st][i] = v;
                    tmax = fmaxf(tmax, v);
                }
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float mnew = fmaxf(mrow, tmax);
            const float muse = (mnew == -INFINITY) ? 0.f : mnew;
            const float alpha = exp2f(mrow - muse);
            float psum = 0.f;
#pragma unroll
            for (int st = 0; st < NST; ++st) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = exp2f(s[st][i] - muse);
                    s[st][i] = pv;
                    psum += pv;
                }
            }
            psum += __shfl_xor(psum, 16);
            psum += __shfl_xor(psum, 32);
            lrow = lrow * alpha + psum;
            mrow = mnew;
#pragma unroll
            for (int nt = 0; nt < 32; ++nt) acc[nt] *= alpha;

            // ---- O^T += V^T P^T
            if constexpr (NST == 1) {
                s16x4 pb;
#pragma unroll
                for (int e = 0; e < 4; ++e) pb[e] = (short)bf16_bits_rne(s[0][e]);
#pragma unroll
                for (int nt = 0; nt < 32; ++nt) {
                    const int d = 16 * nt + c16;
                    s16x4 va;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = tok0 + 4 * g + e;
                        va[e] = *(const short*)(buf + r * kLdsRow + 2 * d);
                    }
                    acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[nt], 0, 0, 0);
                    if ((nt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int kp = 0; kp < NST / 2; ++kp) {
                    s16x8 pb;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pb[e] = (short)bf16_bits_rne(s[2 * kp][e]);
                        pb[e + 4] = (short)bf16_bits_rne(s[2 * kp + 1][e]);
                    }
#pragma unroll
                    for (int nt = 0; nt < 32; ++nt) {
                        const int d = 16 * nt + c16;
                        s16x8 va;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int r = tok0 + 16 * (2 * kp + (e >> 2)) + 4 * g + (e & 3);
                            va[e] = *(const short*)(buf + r * kLdsRow + 2 * d);
                        }
                        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va),
                                                                          __builtin_bit_cast(bf16x8, pb), acc[nt], 0, 0, 0);
                        if ((nt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        }
        __syncthreads();     // every wave is done with the block buffers

        // ---- merge the token slices and write the segment's result
        const int nsplit = p.splits[b + 1] - p.splits[b];
        const int slot = p.splits[b] + split;
        if constexpr (NK == 1) {
            const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
            if (nsplit == 1) {
                uint16_t* o = p.out + ((size_t)b * p.rows_total + myrow) * kDv + 4 * g;
#pragma unroll
                for (int nt = 0; nt < 32; ++nt) {
                    ushort4 v;
                    v.x = bf16_bits_rne(acc[nt][0] * inv);
                    v.y = bf16_bits_rne(acc[nt][1] * inv);
                    v.z = bf16_bits_rne(acc[nt][2] * inv);
                    v.w = bf16_bits_rne(acc[nt][3] * inv);
                    *(ushort4*)(o + 16 * nt) = v;
                }
            } else {
                float* o = p.part_o + ((size_t)slot * p.rows_total + myrow) * kDv + 4 * g;
#pragma unroll
                for (int nt = 0; nt < 32; ++nt) {
                    *(f32x4*)(o + 16 * nt) = acc[nt] * inv;
                }
            }
            if (g == 0) {
                const float l = lrow > 0.f ? (mrow + __log2f(lrow)) * 0.69314718055994531f : -INFINITY;
                if (nsplit == 1) p.lse[(size_t)b * p.rows_total + myrow] = l;
                else p.part_lse[(size_t)slot * p.rows_total + myrow] = l;
            }
        } else {
            float* stat_m = (float*)smem;                  // [NK][MW]
            float* stat_l = stat_m + NK * MW;              // [NK][MW]
            float* obuf = stat_l + NK * MW;                // [MW][kObufStride]
            const int rloc = rg * 16 + c16;                // row within the workgroup
            if (g == 0) stat_m[kk * MW + rloc] = mrow;
            __syncthreads();
            float mall = -INFINITY;
#pragma unroll
            for (int k2 = 0; k2 < NK; ++k2) mall = fmaxf(mall, stat_m[k2 * MW + rloc]);
            const float f = exp2f(mrow - ((mall == -INFINITY) ? 0.f : mall));
            if (g == 0) stat_l[kk * MW + rloc] = lrow * f;
            float* orow = obuf + rloc * kObufStride + 4 * g;
            if (kk == 0) {
#pragma unroll
                for (int nt = 0; nt < 32; ++nt) *(f32x4*)(orow + 16 * nt) = acc[nt] * f;
            }
            __syncthreads();
#pragma unroll
            for (int k2 = 1; k2 < NK; ++k2) {
                if (kk == k2) {
#pragma unroll
                    for (int nt = 0; nt < 32; ++nt) *(f32x4*)(orow + 16 * nt) += acc[nt] * f;
                }
                __syncthreads();
            }
            // wave (rg, kk) finishes dims [kk*DS, (kk+1)*DS) of rows 16rg..16rg+15
            constexpr int DS = kDv / NK;
            constexpr int PER_ROW = DS / 8;
            for (int idx = lane; idx < 16 * PER_ROW; idx += 64) {
                const int r = rg * 16 + idx / PER_ROW;
                const int d = kk * DS + (idx % PER_ROW) * 8;
                float lt = 0.f;
#pragma unroll
                for (int k2 = 0; k2 < NK; ++k2) lt += stat_l[k2 * MW + r];
                const float inv = lt > 0.f ? 1.f / lt : 0.f;
                const f32x4 v0 = *(const f32x4*)(obuf + r * kObufStride + d) * inv;
                const f32x4 v1 = *(const f32x4*)(obuf + r * kObufStride + d + 4) * inv;
                const int grow = blockIdx.y * MW + r;
                if (nsplit == 1) {
                    s16x8 w;
                    w[0] = bf16_bits_rne(v0[0]); w[1] = bf16_bits_rne(v0[1]);
                    w[2] = bf16_bits_rne(v0[2]); w[3] = bf16_bits_rne(v0[3]);
                    w[4] = bf16_bits_rne(v1[0]); w[5] = bf16_bits_rne(v1[1]);
                    w[6] = bf16_bits_rne(v1[2]); w[7] = bf16_bits_rne(v1[3]);
                    *(s16x8*)(p.out + ((size_t)b * p.rows_total + grow) * kDv + d) = w;
                } else {
                    float* o = p.part_o + ((size_t)slot * p.rows_total + grow) * kDv + d;
                    *(f32x4*)o = v0;
                    *(f32x4*)(o + 4) = v1;
                }
            }
            if (kk == 0 && lane < 16) {
                const int r = rg * 16 + lane;
                float lt = 0.f, mx = -INFINITY;
#pragma unroll
                for (int k2 = 0; k2 < NK; ++k2) {
                    lt += stat_l[k2 * MW + r];
                    mx = fmaxf(mx, stat_m[k2 * MW + r]);
                }
                const float l = lt > 0.f ? (mx + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
                const int grow = blockIdx.y * MW + r;
                if (nsplit == 1) p.lse[(size_t)b * p.rows_total + grow] = l;
                else p.part_lse[(size_t)slot * p.rows_total + grow] = l;
            }
            __syncthreads();   // the merge buffer is the next segment's block buffer
        }
    }
}

// Merge split partials by their log-sum-exp; one wave per (sequence, row).
// Sequences with no block get out = 0, lse = -inf; unsplit ones were written
// by the decode kernel.
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int b = blockIdx.y;
    if (row >= p.rows_total) return;
    const int s0 = p.splits[b];
    const int ns = p.splits[b + 1] - s0;
    if (ns == 1) return;
    uint16_t* o = p.out + ((size_t)b * p.rows_total + row) * kDv + lane * 8;
    float* lo = p.lse + (size_t)b * p.rows_total + row;
    float mx = -INFINITY;
    for (int k = 0; k < ns; ++k) mx = fmaxf(mx, p.part_lse[(size_t)(s0 + k) * p.rows_total + row]);
    if (ns == 0 || mx == -INFINITY) {
        *(uint4*)o = make_uint4(0, 0, 0, 0);
        if (lane == 0) *lo = -INFINITY;
        return;
    }
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    for (int k = 0; k < ns; ++k) {
        const size_t sr = (size_t)(s0 + k) * p.rows_total + row;
        const float w = __expf(p.part_lse[sr] - mx);
        wsum += w;
        const float* src = p.part_o + sr * kDv + lane * 8;
        a0 += *(const f32x4*)src * w;
        a1 += *(const f32x4*)(src + 4) * w;
    }
    const float inv = 1.f / wsum;
    s16x8 w8;
    w8[0] = bf16_bits_rne(a0[0] * inv); w8[1] = bf16_bits_rne(a0[1] * inv);
    w8[2] = bf16_bits_rne(a0[2] * inv); w8[3] = bf16_bits_rne(a0[3] * inv);
    w8[4] = bf16_bits_rne(a1[0] * inv); w8[5] = bf16_bits_rne(a1[1] * inv);
    w8[6] = bf16_bits_rne(a1[2] * inv); w8[7] = bf16_bits_rne(a1[3] * inv);
    *(s16x8*)o = w8;
    if (lane == 0) *lo = mx + __logf(wsum);
}

hipError_t launch_decode(const DecodeParams& p, int num_units, int head_groups, int rows_wg, hipStream_t stream)
{
    dim3 grid(num_units, head_groups);
    switch (rows_wg) {
    case 16: hipLaunchKernelGGL((decode_kernel<1, 4>), grid, dim3(256), 0, stream, p); break;
    case 32: hipLaunchKernelGGL((decode_kernel<2, 4>), grid, dim3(512), 0, stream, p); break;
    case 64: hipLaunchKernelGGL((decode_kernel<4, 2>), grid, dim3(512), 0, stream, p); break;
    case 128: hipLaunchKernelGGL((decode_kernel<8, 1>), grid, dim3(512), 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream)
{
    dim3 grid((p.rows_total + 3) / 4, p.batch);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mla
