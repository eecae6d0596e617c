// Shared definitions of the HIP library: launch shapes, the split-KV plan's
// integer formulas (used by both the device planner and the host planner so
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

// Query rows per workgroup: the largest of 128/64/32/16 dividing s_q*h_q.
// Rows beyond that are covered by more workgroups ("head groups") that read
// the same cache blocks.
inline __host__ __device__ int rows_per_wg(int rows_total)
{
    if (rows_total % 128 == 0) return 128;
    if (rows_total % 64 == 0) return 64;
    if (rows_total % 32 == 0) return 32;
    return 16;
}

// Fixed cost of one (unit, sequence) segment, in cache blocks: loading the
// queries and writing a partial result costs about this much traffic.
inline __host__ __device__ int segment_cost(int rows_wg) { return 1 + rows_wg / 32; }

inline __host__ __device__ int blocks_of(int len) { return len > 0 ? (len + kPage - 1) / kPage : 0; }

// Plan geometry: the blocks of the batch, in (sequence, block) order, sit on a
// "cost line". Sequence b starts at P[b] (exclusive prefix sum of cost_b =
// n_b + kappa for non-empty sequences, 0 otherwise); its block j sits at
// P[b] + kappa + j. Unit u owns the blocks whose position lies in
// [u*W, (u+1)*W), W = ceil(C / G) with C = P[batch].
inline __host__ __device__ int plan_width(int total_cost, int num_units)
{
    int w = (total_cost + num_units - 1) / num_units;
    return w > 0 ? w : 1;
}

// First block (b, j) whose position is >= T. P has batch+1 entries.
// Returns b = batch, j = 0 when no block qualifies.
inline __host__ __device__ void plan_locate(const int* P, int batch, int kappa, int T, int* b_out, int* j_out)
{
    // smallest b with P[b+1] > T (such a b always has blocks: see plan notes)
    int lo = 0, hi = batch;                     // answer in [lo, hi]
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (P[mid + 1] > T) hi = mid; else lo = mid + 1;
    }
    if (lo >= batch) { *b_out = batch; *j_out = 0; return; }
    int j = T - P[lo] - kappa;
    *b_out = lo;
    *j_out = j > 0 ? j : 0;
}

// Units touching sequence b (0 when it has no block).
inline __host__ __device__ int plan_splits(int Pb, int nb, int kappa, int W)
{
    if (nb <= 0) return 0;
    return (Pb + kappa + nb - 1) / W - (Pb + kappa) / W + 1;
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
