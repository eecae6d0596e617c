// Device-side building blocks shared by the decode kernels (gfx950): vector
// types, direct global->LDS copies, explicit wait counts, scalar loads of
// wave-uniform values, cross-lane reductions and LDS access helpers.
#pragma once

#include "mla_common.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) s16x8 lds_s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_rw;

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

// One 16-byte global->LDS copy per lane from a wave-uniform base plus a
// per-lane 32-bit byte offset (the scalar-base form of the copy).
__device__ __forceinline__ void dma16s(const unsigned char* sbase, unsigned voff, unsigned lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds_addr)
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

// Load of a wave-uniform int through the constant address space: the
// compiler emits a scalar load counted by lgkmcnt and waits for it only where
// the value is first used, so it can be issued well ahead of that use. Only
// for buffers that no one writes while the kernel runs.
__device__ __forceinline__ int cload(const int32_t* ptr)
{
    return *(const __attribute__((address_space(4))) int32_t*)(uintptr_t)ptr;
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

// ---- FP8 cache staging (both FP8 decode kernels). A 32-token slot is 1216
// chunks of 16 B (19 one-KB copies): rows 0-15 of E4M3 codes at chunk 37 r,
// rows 16-31 at 37 r + 1 (576 B of codes + one pad chunk per row; the extra
// chunk keeps rows r and r + 16 in different banks), then the 32 row scales
// at chunk 1185.
constexpr int kF8Chunks = 37;                        // chunks per LDS row: 36 of codes + 1 pad
constexpr int kF8Row16 = 16 * kF8Chunks + 1;         // chunk position of row 16
constexpr int kF8Scale = 2 * 16 * kF8Chunks + 1;     // chunk position of the 32 row scales
constexpr int kF8SlotB = 19 * 1024;                  // one 32-token slot

__device__ __forceinline__ unsigned f8_row(int r) { return 16u * (unsigned)(kF8Chunks * r + (r >> 4)); }

// Eight E4M3 codes -> eight bf16 values, exactly (every E4M3 value is a bf16 value).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(u32x2 raw)
{
    const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.f, false);
    const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.f, true);
    const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.f, false);
    const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.f, true);
    return bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

__device__ __forceinline__ unsigned short bf16_rne(float f)
{
    unsigned u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (unsigned short)(u >> 16);
}

// A block-table entry as the decode kernels use it: entries outside [0, nblocks)
// read block 0 instead, so a table that breaks the contract never makes a
// kernel read outside the cache (the sequence's result is then unspecified).
__device__ __forceinline__ int safe_page(int page, int64_t nblocks) { return (page >= 0 && page < nblocks) ? page : 0; }

__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b)
{
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Entries j .. j + 63 of sequence b's block-table row, entry j + i in lane i
// (0 past the row): a vector load, so its wait is counted with the block
// copies rather than with the LDS operations.
__device__ __forceinline__ int table_window(const DecodeParams& p, int b, int j, int lane)
{
    const int jj = j + lane;
    return jj < p.max_blocks ? p.block_table[(size_t)b * p.max_blocks + jj] : 0;
}

// ---------------------------------------------------------------- units of the cost-line plan

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

// Chunk permutation of a row r of a 32-row block half in LDS (64- and 128-row
// kernels; rows are unpadded): chunk c is stored at position c ^ f(r) with
// f(r) = ((r << 1) ^ (r >> 2)) mod 16, chunks 64-71 by the low three bits of
// f only (so they stay in 64-71); the map is its own inverse. The LDS serves
// a 16-byte read 16 lanes per cycle from 16 groups of four banks, and row r
// starts in group 8r mod 16: with this f the 16 rows of a K fragment read
// (any chunk) and the 4 rows x 4 chunks of a V^T transpose read each fall in
// 16 different groups.
__device__ __forceinline__ int swz_f(int r) { return ((r << 1) ^ (r >> 2)) & 15; }
__device__ __forceinline__ int swz_chunk(int r, int c) { return c < 64 ? (c ^ swz_f(r)) : (c ^ (swz_f(r) & 7)); }
__device__ __forceinline__ unsigned swz(int r, int c) { return (unsigned)(r * kRowBytes + (swz_chunk(r, c) << 4)); }

}  // namespace mla
