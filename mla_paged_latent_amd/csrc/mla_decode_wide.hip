// MLA decode, wide kernel (gfx950): 64 query rows per workgroup on
// v_mfma_f32_32x32x16_bf16. Built with the VGPR form of the matrix ops so the
// output accumulators live in VGPRs, where the online-softmax rescale can
// scale them in place (AGPR accumulators would need a copy through VGPRs).
#include "mla_device.h"

namespace mla {

// ---------------------------------------------------------------- wide kernel
//
// 64 query rows per workgroup, four waves: wave = 2 rg + kh holds rows
// [32 rg, 32 rg + 32) of the workgroup; kh picks the half of the work it does.
// QK^T: wave kh contracts cached columns [288 kh, 288 kh + 288) (its 72-register
// half of Q); the two partial S^T tiles of a row group are summed through LDS.
// PV: wave kh accumulates output dims [256 kh, 256 kh + 256) (128 registers).
// Both waves of a row group run the same softmax on the same S and so keep
// identical running max and sum. The four waves share a ring of four 32-token
// slots. Within a sequence the work is software pipelined: while slot n's
// exponentials and PV run, slot n+1's QK^T is issued (the exponentials sit
// between its matrix ops) and slots n+2, n+3 are in flight. Slots hold rows of
// 1152 B with chunk c of row r at position c ^ (r % 8), which with the token
// permutation keeps b128 and transpose reads conflict free.

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
    s.L = cload(p.seqlens + b);
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
    const float c = p.scale_log2;

    Segment is = next_segment(p, b0, b0, j0, b1, j1);      // copy cursor
    if (is.b >= p.batch) return;
    int itok = is.tb;
    // page of the next slot to copy, loaded one slot ahead of its use
    int ipage = cload(p.block_table + (size_t)is.b * p.max_blocks + (itok >> 6));
    Segment cs = is;                                        // compute cursor

    // This wave's 9 copies of a slot: copy i = wave + 4k, lane l fills LDS
    // position s of row r (72 r + s = 64 i + l) with chunk s ^ (r % 8).
    unsigned dma_off[9];
    int dma_row[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const int q = (wave + 4 * k) * 64 + lane;
        const int r = q / kChunks;
        dma_row[k] = r;
        dma_off[k] = (unsigned)(r * kRowBytes + (((q - r * kChunks) ^ (r & 7)) << 4));
    }
    int n_issued = 0;
    // The next slot to copy: global base, LDS base of this wave's copies, and
    // how many of its 32 rows are real (rows past the end are copied from row
    // 0: finite data, masked later).
    struct Copy {
        const unsigned char* gbase;
        unsigned slot;
        int valid;
    };
    auto copy_begin = [&]() {
        Copy cp;
        cp.gbase = (const unsigned char*)p.kcache + (size_t)ipage * kPageBytes + (size_t)(itok & 63) * kRowBytes;
        cp.slot = lds0 + (unsigned)(n_issued & 3) * kSlotB + (unsigned)wave * 1024u;
        cp.valid = is.te - itok;
        return cp;
    };
    auto copy_one = [&](const Copy& cp, int k) {
        const unsigned off = cp.valid >= 32 || dma_row[k] < cp.valid ? dma_off[k]
                                                                     : dma_off[k] - (unsigned)(dma_row[k] * kRowBytes);
        dma16s(cp.gbase, off, cp.slot + 4096u * k);
    };
    auto copy_end = [&]() {
        ++n_issued;
        itok += 32;
        if (itok >= is.te) {
            is = next_segment(p, is.b + 1, b0, j0, b1, j1);
            itok = is.tb;
        }
        if (is.b < p.batch && (itok & 63) == 0) ipage = cload(p.block_table + (size_t)is.b * p.max_blocks + (itok >> 6));
    };
    auto issue = [&]() {
        const Copy cp = copy_begin();
#pragma unroll
        for (int k = 0; k < 9; ++k) copy_one(cp, k);
        copy_end();
    };
    // wait until slot m has landed (for this wave's copies), then sync the
    // workgroup; the ring may then be refilled while slot `oldest` stays untouched
    auto arrive = [&](int m) {
        const int later = n_issued - 1 - m;
        if (later <= 0) MLA_WAIT_VM(0);
        else if (later == 1) MLA_WAIT_VM(9);
        else if (later == 2) MLA_WAIT_VM(18);
        else MLA_WAIT_VM(27);
        wg_barrier();
    };
    for (int k = 0; k < 3 && is.b < p.batch; ++k) issue();

    // QK^T A operand rows: token row tokA; for k-step ks = 4 j + m its chunk is
    // 36 kh + 2 ks + h, stored at ((36 kh + h + 2 m) ^ (tokA % 8)) + 8 j
    const int tokA = token_of_row(r32);
    unsigned k_off[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        k_off[m] = (unsigned)(tokA * kRowBytes + (((36 * kh + h + 2 * m) ^ (tokA & 7)) << 4));
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
                const int ch = 32 * kh + 4 * par + 2 * dh + ((i16 & 3) >> 1);
                v_off[kp][half][par] = swz(r, ch) + 8u * (unsigned)(i16 & 1);
            }
    // partial S^T tiles: element group j of lane l at 1024 j + 16 l of the wave's 4 KB
    const unsigned xmine = lds0 + 4 * kSlotB + (unsigned)(wave * 4096 + lane * 16);
    const unsigned xother = lds0 + 4 * kSlotB + (unsigned)((wave ^ 1) * 4096 + lane * 16);

    int n = 0;                                              // slot being computed
    while (cs.b < p.batch) {
        // new segment: this wave's half of its 32 query rows, fresh softmax state
        bf16x8 qf[18];
        {
            const uint16_t* qrow = p.q + ((size_t)cs.b * p.rows_total + row) * kDqk + 288 * kh + 8 * h;
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, *(const s16x8*)(qrow + 16 * ks));
            settle_loads();
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) asm volatile("" : "+a"(qf[ks]));
        }
        f32x16 acc[8];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[nt][i] = 0.f;
        float mrun = -INFINITY, lrun = 0.f;
        const int lim = min(cs.te, p.causal ? cs.L - (p.s_q - 1 - iq) : cs.L);
        // lane 0 holds the wave's first row, whose visible prefix is the shortest
        const int lim_lo = __builtin_amdgcn_readfirstlane(lim);

        // K operand of k-step ks of slot base sb
        auto load_k = [&](unsigned sb, int ks) {
            return lds_load16(sb + k_off[ks & 3] + 128u * (unsigned)(ks >> 2));
        };
        // partial S^T of slot m over this wave's column half, K loads kept 4 ahead
        auto qk = [&](int m) {
            const unsigned sb = lds0 + (unsigned)(m & 3) * kSlotB;
            f32x16 s;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = 0.f;
            s16x8 kv[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) kv[ks] = load_k(sb, ks);
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) {
                __builtin_amdgcn_sched_barrier(0);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv[ks & 3]), qf[ks], s, 0, 0, 0);
                if (ks + 4 < 18) kv[ks & 3] = load_k(sb, ks + 4);
            }
            __builtin_amdgcn_sched_barrier(0);
            return s;
        };
        // the same, with the exponentials of the previous slot's softmax placed
        // between the matrix ops (they are independent of them)
        // (and, when `copy` is set, this wave's nine copies of the next ring
        // slot spread over the matrix ops, so their issue never stalls the
        // wave for long)
        auto qk_exp = [&](int m, const float* sv, float cs, float muse, float* pv, bool copy, const Copy& cp) {
            const unsigned sb = lds0 + (unsigned)(m & 3) * kSlotB;
            f32x16 s;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = 0.f;
            s16x8 kv[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) kv[ks] = load_k(sb, ks);
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) {
                __builtin_amdgcn_sched_barrier(0);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv[ks & 3]), qf[ks], s, 0, 0, 0);
                if (ks + 4 < 18) kv[ks & 3] = load_k(sb, ks + 4);
                if (ks < 16) pv[ks] = __builtin_amdgcn_exp2f(fmaf(sv[ks], cs, -muse));
                if ((ks & 1) && copy) copy_one(cp, ks >> 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            return s;
        };
        // exchange partial tiles within the row group; returns the full S^T
        auto exchange = [&](f32x16 s) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *(lds_f32x4*)(uintptr_t)(xmine + 1024 * j) = f32x4{s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]};
            wg_barrier();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 o = *(const lds_f32x4*)(uintptr_t)(xother + 1024 * j);
                s[4 * j] += o[0]; s[4 * j + 1] += o[1]; s[4 * j + 2] += o[2]; s[4 * j + 3] += o[3];
            }
            return s;
        };
        // first half of the online softmax of S^T for tokens [t0, t0 + 32):
        // element i is token t0 + token_of_row(8(i/4) + 4h + i%4) of query row
        // r32. Scales and masks the scores into sv, raises the running max
        // (rescaling O and the sum) and returns the max the exponentials use.
        // Without masking (and with a positive scale) sv keeps the raw scores
        // and `cs` returns the scale; with masking sv holds scaled, masked
        // scores and cs = 1. The exponentials take exp2(sv * cs - max).
        auto prepare = [&](const f32x16& s, int t0, float* sv, float& cs) {
            float m4[4];
            if (t0 + 32 <= lim_lo && c > 0.f) {
#pragma unroll
                for (int i = 0; i < 16; ++i) sv[i] = s[i];
                cs = c;
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int t = t0 + token_of_row(8 * (i >> 2) + 4 * h + (i & 3));
                    sv[i] = (t < lim) ? s[i] * c : -INFINITY;
                }
                cs = 1.f;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                m4[j] = fmaxf(fmaxf(sv[4 * j], sv[4 * j + 1]), fmaxf(sv[4 * j + 2], sv[4 * j + 3]));
            float tmax = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])) * cs;   // the scaled max (cs > 0)
            tmax = xor32_max(tmax);
            const bool need = tmax > mrun + kLazyTau;
            if (wave_any(need)) {
                const float mnew = need ? tmax : mrun;
                const float alpha = need ? __builtin_amdgcn_exp2f(mrun - mnew) : 1.f;
                lrun *= alpha;
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) acc[nt] *= alpha;
                mrun = mnew;
            }
            return mrun == -INFINITY ? 0.f : mrun;
        };
        // second half: row sums and P^T as the bf16 B operands of the two PV k-steps
        auto finish = [&](const float* pv, bf16x8* pb) {
            float q4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) q4[j] = (pv[4 * j] + pv[4 * j + 1]) + (pv[4 * j + 2] + pv[4 * j + 3]);
            lrun += xor32_sum((q4[0] + q4[1]) + (q4[2] + q4[3]));
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) {
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(pv[8 * kp + 2 * e], pv[8 * kp + 2 * e + 1]);
                pb[kp] = __builtin_bit_cast(bf16x8, w);
            }
        };
        // O^T += V^T P^T over the slot's two 16-token k-steps, this wave's 256
        // dims; V^T operands kept 4 matrix ops ahead
        auto pv_step = [&](int m, const bf16x8* pb) {
            const unsigned sb = lds0 + (unsigned)(m & 3) * kSlotB;
            s16x4 va[4][2];
            auto load_v = [&](int k, s16x4* d) {
                const int nt = k >> 1, kp = k & 1;
                const unsigned off = 128u * (unsigned)(nt >> 1);
                d[0] = lds_tr4(sb + v_off[kp][0][nt & 1] + off);
                d[1] = lds_tr4(sb + v_off[kp][1][nt & 1] + off);
            };
#pragma unroll
            for (int k = 0; k < 4; ++k) load_v(k, va[k]);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                __builtin_amdgcn_sched_barrier(0);
                const int nt = k >> 1, kp = k & 1;
                const s16x4 lo = va[k & 3][0], hi = va[k & 3][1];
                const s16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb[kp], acc[nt], 0, 0, 0);
                if (k + 4 < 16) load_v(k + 4, va[k & 3]);
            }
            __builtin_amdgcn_sched_barrier(0);
        };

        // first slot of the segment; afterwards each step issues the next
        // slot's QK^T beside this slot's exponentials, then this slot's PV
        arrive(n);
        while (is.b < p.batch && n_issued < n + 4) issue();
        f32x16 s = exchange(qk(n));
        for (int t0 = cs.tb;; t0 += 32) {
            const bool more = t0 + 32 < cs.te;
            float sv[16], pv[16], scl;
            const float muse = prepare(s, t0, sv, scl);
            f32x16 s_next;
            if (more) {
                arrive(n + 1);
                // slot n is still read by this step's PV: refill only up to n + 3
                const bool copy = is.b < p.batch && n_issued < n + 4;
                const Copy cp = copy_begin();
                s_next = qk_exp(n + 1, sv, scl, muse, pv, copy, cp);
                if (copy) copy_end();
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], scl, -muse));
            }
            bf16x8 pb[2];
            finish(pv, pb);
            pv_step(n, pb);
            ++n;
            if (!more) break;
            s = exchange(s_next);
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
                    u32x2 v;
                    v[0] = pack_bf16x2(acc[nt][4 * j + 0] * inv, acc[nt][4 * j + 1] * inv);
                    v[1] = pack_bf16x2(acc[nt][4 * j + 2] * inv, acc[nt][4 * j + 3] * inv);
                    *(u32x2*)(o + 32 * nt + 8 * j) = v;
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

hipError_t launch_wide(const DecodeParams& p, dim3 grid, hipStream_t stream)
{
    hipLaunchKernelGGL(decode_wide_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mla
