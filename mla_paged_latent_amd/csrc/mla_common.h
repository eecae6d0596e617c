// Shared definitions of the HIP library: shapes, launch geometry, the split-KV
// plan's integer formulas (used by the device planner and the host planner so
// the two agree bit for bit) and the kernel parameter blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kDqk = 576;          // cached row: 512 latent + 64 rope columns
constexpr int kDv = 512;           // value = first 512 columns of the row
constexpr int kPage = 64;          // tokens per cache block
constexpr int kRowBytes = kDqk * 2;
constexpr int kPageBytes = kPage * kRowBytes;   // 73,728 B, contiguous in HBM
constexpr int kMetaInts = 8;
constexpr int kMaxRows = 1024;     // largest s_q*h_q accepted

// Query rows per workgroup: 64 when s_q*h_q is a multiple of 64 (the
// 32x32-MFMA kernel: two row groups of 32, each split over two waves), else
// 16 (the streaming kernel, every wave holds all 16 rows). Rows beyond that
// are covered by more workgroups ("head groups") reading the same blocks.
inline __host__ __device__ int rows_per_wg(int rows_total)
{
    return rows_total % 64 == 0 ? 64 : 16;
}

// Two plan shapes.
//  * Streaming kernel (16 rows): every unit is one sequence's run of blocks.
//    W = ceil(total_blocks / G) blocks at most per unit; sequence b is cut into
//    ns_b = ceil(n_b / W) near-equal runs. Units number sum(ns_b) <= G + B.
//  * 64-row kernel: blocks of the batch, in (sequence, block) order, sit on a
//    cost line where sequence b starts at P[b] and pays a fixed segment cost
//    kappa before its first block; unit u owns the blocks whose position lies
//    in [u*W, (u+1)*W), W = ceil(C / G). A unit may span several sequences.
inline __host__ __device__ bool plan_by_sequence(int rows_wg) { return rows_wg < 64; }

// Fixed cost of one (unit, sequence) segment of the 64-row kernel, in cache
// blocks: reloading 64 query rows and writing 64 result rows costs about this
// much traffic.
constexpr int kSegmentCost = 4;

inline __host__ __device__ int blocks_of(int len) { return len > 0 ? (len + kPage - 1) / kPage : 0; }

inline __host__ __device__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

inline __host__ __device__ int plan_width(int total_cost, int num_units)
{
    int w = ceil_div(total_cost, num_units);
    return w > 0 ? w : 1;
}

// Cost-line plan: first block (b, j) whose position is >= T. P has batch+1
// entries. Returns b = batch, j = 0 when no block qualifies.
inline __host__ __device__ void plan_locate(const int* P, int batch, int kappa, int T, int* b_out, int* j_out)
{
    // smallest b with P[b+1] > T; such a b always has blocks (an empty sequence
    // has P[b+1] == P[b], so an earlier b would already qualify)
    int lo = 0, hi = batch;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (P[mid + 1] > T) hi = mid; else lo = mid + 1;
    }
    if (lo >= batch) { *b_out = batch; *j_out = 0; return; }
    int j = T - P[lo] - kappa;
    *b_out = lo;
    *j_out = j > 0 ? j : 0;
}

// Cost-line plan: units touching sequence b (0 when it has no block).
inline __host__ __device__ int plan_splits(int Pb, int nb, int kappa, int W)
{
    if (nb <= 0) return 0;
    return (Pb + kappa + nb - 1) / W - (Pb + kappa) / W + 1;
}

// Per-sequence plan: sequence b's split k covers blocks [k*n/ns, (k+1)*n/ns).
inline __host__ __device__ int split_begin(int n, int ns, int k) { return (int)(((long long)k * n) / ns); }

// Per-sequence plan: unit u -> (sequence, split) given prefix sums Q of the
// split counts (Q[0] = 0, Q[batch] = total units). Returns b = batch if u is
// past the last unit.
inline __host__ __device__ int plan_owner(const int* Q, int batch, int u)
{
    // largest b with Q[b] <= u and Q[b+1] > u
    int lo = 0, hi = batch;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (Q[mid + 1] > u) hi = mid; else lo = mid + 1;
    }
    return lo;
}

struct DecodeParams {
    const uint16_t* q;          // [B, rows_total, 576] bf16 (rows = s_q*h_q, i-major)
    const uint16_t* kcache;     // [nblocks, 64, 576] bf16
    const int32_t* block_table; // [B, max_blocks]
    const int32_t* seqlens;     // [B]
    const int32_t* meta;        // [G, 8]
    const int32_t* splits;      // [B+1] prefix sums
    uint16_t* out;              // [B, rows_total, 512] bf16
    float* lse;                 // [B, rows_total]
    float* part_o;              // [slots, rows_total, 512] fp32
    float* part_lse;            // [slots, rows_total]
    int64_t nblocks;
    int max_blocks;
    int batch;
    int s_q;
    int h_q;
    int rows_total;
    int causal;
    float scale_log2;           // softmax_scale * log2(e)
    // sparse decode only: "sequence" b is new token b % sq_real of sequence
    // b / sq_real, and its token t is cached position indices[b * topk + t]
    const int32_t* indices;
    int topk;
    int sq_real;
    // FP8 decode only: kcache holds E4M3 codes [nblocks, 64, 576] and kscale
    // the float32 scale of each cached row [nblocks, 64]
    const float* kscale;
};

struct CombineParams {
    const int32_t* splits;      // [B+1]
    const float* part_o;
    const float* part_lse;
    uint16_t* out;
    float* lse;
    int batch;
    int rows_total;
};

}  // namespace mla
