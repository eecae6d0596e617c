// Split-KV tile plan for variable-length decode batches.
//
// The pages state only that the decode kernel is tuned for serving sequences
// of varying length (GeekNews release note, id.news.hada.io; FlashMLA
// explainer section 2.4 on padding waste). The two plan shapes below are this
// library's own (see mla_common.h): per-sequence runs for the streaming
// kernel, a cost line cut into equal parts for the 64-row kernel. In both,
// every cache block belongs to exactly one unit and a unit's blocks are
// contiguous in (sequence, block) order.
//
// The device planner (one workgroup) and the host planner evaluate the same
// integer formulas, so their outputs agree bit for bit.
#include "mla_common.h"

namespace mla {

constexpr int kPlanThreads = 1024;       // largest workgroup; small batches launch 256 threads

// Threads of the planner for a batch: one workgroup either way; a small batch
// finishes sooner with fewer waves to synchronise, a large one needs them all.
inline int plan_threads(int batch) { return batch <= 1024 ? 256 : kPlanThreads; }

// Inclusive prefix sum across the 64 lanes of a wave, in registers with DPP:
// shifts by 1, 2, 4 and 8 within each 16-lane row (lanes shifted in from
// outside the row add 0), then the total of row 0 is added to row 1 and that
// of row 2 to row 3 (row_bcast:15), then the total of rows 0-1 to rows 2-3
// (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_scan(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2, 3
    return x;
}

// Inclusive prefix sum of a[0..n) in LDS by one workgroup (blockDim.x threads):
// every thread sums a contiguous chunk, the chunk sums are scanned within each
// wave and across the waves' totals (carry[], one int per wave), then every
// thread rewrites its chunk. Two workgroup barriers.
__device__ void block_inclusive_scan(int* a, int n, int* carry)
{
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int wave = tid >> 6;
    const int per = (n + nthr - 1) / nthr;
    const int lo = tid * per;
    const int hi = min(lo + per, n);
    int local = 0;
    for (int k = lo; k < hi; ++k) local += a[k];
    const int incl = wave_inclusive_scan(local);
    if ((tid & 63) == 63) carry[wave] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < wave; ++w) run += carry[w];
    for (int k = lo; k < hi; ++k) {
        run += a[k];
        a[k] = run;
    }
    __syncthreads();
}

// Row u of the plan: {b_begin, blk_begin, b_end, blk_end, split index of the
// first segment, cache_seqlens[b_begin], partial slot of the first segment
// (num_splits[b_begin] + split index), number of splits of b_begin}. The last
// three are zero for an empty unit; they spare the decode kernel dependent
// loads at its start and end.
__device__ __host__ inline void write_meta(int32_t* m, int b0, int j0, int b1, int j1, int split, int len,
                                           int first_slot, int nsplit)
{
    m[0] = b0; m[1] = j0; m[2] = b1; m[3] = j1; m[4] = split;
    m[5] = len; m[6] = first_slot; m[7] = nsplit;
}

// Per-sequence plan: first block of split k of a sequence of n blocks cut
// into ns runs (split_begin), in 32-bit arithmetic when k * n fits.
__device__ __forceinline__ int split_begin_dev(int n, int ns, int k)
{
    const long long kn = (long long)k * n;
    return kn < 0x7FFFFFFF ? (int)kn / ns : (int)(kn / ns);
}

// Batches of at most 64 sequences: every wave builds the prefix sums of its
// own from one sequence per lane (wave scans, a private copy in LDS with the
// lengths), so the workgroup needs no barrier and the units' rows need no
// second global load; threads then fill the rows as below.
__device__ void plan_small(const int32_t* __restrict__ seqlens, int batch, int rows_wg, int num_units,
                           int32_t* __restrict__ meta, int32_t* __restrict__ splits, int* smem)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    int* P = smem + (tid >> 6) * 3 * 65;                    // [65]: this wave's copy
    int* NS = P + 65;                                       // [65]
    int* LEN = NS + 65;                                     // [64]: cache_seqlens
    const int len = lane < batch ? seqlens[lane] : 0;
    const int nb = blocks_of(len);
    const bool by_seq = plan_by_sequence(rows_wg);
    const int kappa = by_seq ? 0 : kSegmentCost;
    const int cost = nb > 0 ? nb + kappa : 0;
    const int pin = wave_inclusive_scan(cost);
    const int total = __builtin_amdgcn_readlane(pin, 63);
    const int W = by_seq ? plan_width(total, num_units - batch) : plan_width(total, num_units);
    const int ns = lane < batch ? (by_seq ? ceil_div(nb, W) : plan_splits(pin - cost, nb, kappa, W)) : 0;
    const int nsin = wave_inclusive_scan(ns);
    P[lane + 1] = pin;
    NS[lane + 1] = nsin;
    LEN[lane] = len;
    if (lane == 0) { P[0] = 0; NS[0] = 0; }
    // a wave's LDS accesses complete in order: once its stores are issued, its
    // lanes read each other's entries (the asm keeps the compiler from moving
    // loads above them)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (tid < 64)
        for (int i = lane; i <= batch; i += 64) splits[i] = NS[i];
    for (int u = tid; u < num_units; u += blockDim.x) {
        int32_t* m = meta + (size_t)u * kMetaInts;
        if (by_seq) {
            const int b = plan_owner(NS, batch, u);
            if (b >= batch) { write_meta(m, batch, 0, batch, 0, 0, 0, 0, 0); continue; }
            const int n = P[b + 1] - P[b];
            const int nsb = NS[b + 1] - NS[b];
            const int k = u - NS[b];
            write_meta(m, b, split_begin_dev(n, nsb, k), b, split_begin_dev(n, nsb, k + 1), k, LEN[b], NS[b] + k, nsb);
        } else {
            int b0, j0, b1, j1;
            plan_locate(P, batch, kappa, u * W, &b0, &j0);
            plan_locate(P, batch, kappa, (u + 1) * W, &b1, &j1);
            const bool any = b0 < batch && (b0 != b1 || j0 != j1);
            const int split = any ? u - (P[b0] + kappa) / W : 0;
            write_meta(m, b0, j0, b1, j1, split, any ? LEN[b0] : 0, any ? NS[b0] + split : 0,
                       any ? NS[b0 + 1] - NS[b0] : 0);
        }
    }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ seqlens, int batch,
                                                             int rows_wg, int num_units,
                                                             int32_t* __restrict__ meta,
                                                             int32_t* __restrict__ splits)
{
    extern __shared__ int plan_smem[];
    int* P = plan_smem;                  // [batch + 1]
    int* NS = P + (batch + 1);           // [batch + 1]
    int* carry = NS + (batch + 1);       // [kPlanThreads / 64]
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;

    if (batch <= 64) {
        plan_small(seqlens, batch, rows_wg, num_units, meta, splits, plan_smem);
        return;
    }
    if (plan_by_sequence(rows_wg)) {
        // P = prefix sums of the block counts
        for (int b = tid; b < batch; b += nthr) P[b + 1] = blocks_of(seqlens[b]);
        if (tid == 0) P[0] = 0;
        __syncthreads();
        block_inclusive_scan(P + 1, batch, carry);
        const int W = plan_width(P[batch], num_units - batch);
        for (int b = tid; b < batch; b += nthr) NS[b + 1] = ceil_div(P[b + 1] - P[b], W);
        if (tid == 0) NS[0] = 0;
        __syncthreads();
        block_inclusive_scan(NS + 1, batch, carry);
        for (int b = tid; b <= batch; b += nthr) splits[b] = NS[b];
        for (int u = tid; u < num_units; u += nthr) {
            int32_t* m = meta + (size_t)u * kMetaInts;
            int b = plan_owner(NS, batch, u);
            if (b >= batch) { write_meta(m, batch, 0, batch, 0, 0, 0, 0, 0); continue; }
            int n = P[b + 1] - P[b];
            int ns = NS[b + 1] - NS[b];
            int k = u - NS[b];
            write_meta(m, b, split_begin(n, ns, k), b, split_begin(n, ns, k + 1), k, seqlens[b], NS[b] + k, ns);
        }
        return;
    }

    const int kappa = kSegmentCost;
    for (int b = tid; b < batch; b += nthr) {
        int nb = blocks_of(seqlens[b]);
        P[b + 1] = nb > 0 ? nb + kappa : 0;
    }
    if (tid == 0) P[0] = 0;
    __syncthreads();
    block_inclusive_scan(P + 1, batch, carry);

    const int W = plan_width(P[batch], num_units);
    for (int b = tid; b < batch; b += nthr) {
        int cost = P[b + 1] - P[b];
        int nb = cost > 0 ? cost - kappa : 0;
        NS[b + 1] = plan_splits(P[b], nb, kappa, W);
    }
    if (tid == 0) NS[0] = 0;
    __syncthreads();
    block_inclusive_scan(NS + 1, batch, carry);
    for (int b = tid; b <= batch; b += nthr) splits[b] = NS[b];

    for (int u = tid; u < num_units; u += nthr) {
        int b0, j0, b1, j1;
        plan_locate(P, batch, kappa, u * W, &b0, &j0);
        plan_locate(P, batch, kappa, (u + 1) * W, &b1, &j1);
        const bool any = b0 < batch && (b0 != b1 || j0 != j1);
        int split = any ? u - (P[b0] + kappa) / W : 0;
        write_meta(meta + (size_t)u * kMetaInts, b0, j0, b1, j1, split, any ? seqlens[b0] : 0,
                   any ? NS[b0] + split : 0, any ? NS[b0 + 1] - NS[b0] : 0);
    }
}

void plan_host(const int32_t* seqlens, int batch, int rows_wg, int num_units, int32_t* meta, int32_t* splits)
{
    int* P = new int[batch + 1];
    P[0] = 0;
    if (plan_by_sequence(rows_wg)) {
        for (int b = 0; b < batch; ++b) P[b + 1] = P[b] + blocks_of(seqlens[b]);
        const int W = plan_width(P[batch], num_units - batch);
        splits[0] = 0;
        for (int b = 0; b < batch; ++b) splits[b + 1] = splits[b] + ceil_div(P[b + 1] - P[b], W);
        for (int u = 0; u < num_units; ++u) {
            int32_t* m = meta + (size_t)u * kMetaInts;
            int b = plan_owner(splits, batch, u);
            if (b >= batch) { write_meta(m, batch, 0, batch, 0, 0, 0, 0, 0); continue; }
            int n = P[b + 1] - P[b];
            int ns = splits[b + 1] - splits[b];
            int k = u - splits[b];
            write_meta(m, b, split_begin(n, ns, k), b, split_begin(n, ns, k + 1), k, seqlens[b], splits[b] + k, ns);
        }
        delete[] P;
        return;
    }
    const int kappa = kSegmentCost;
    for (int b = 0; b < batch; ++b) {
        int nb = blocks_of(seqlens[b]);
        P[b + 1] = P[b] + (nb > 0 ? nb + kappa : 0);
    }
    const int W = plan_width(P[batch], num_units);
    splits[0] = 0;
    for (int b = 0; b < batch; ++b) {
        int cost = P[b + 1] - P[b];
        int nb = cost > 0 ? cost - kappa : 0;
        splits[b + 1] = splits[b] + plan_splits(P[b], nb, kappa, W);
    }
    for (int u = 0; u < num_units; ++u) {
        int b0, j0, b1, j1;
        plan_locate(P, batch, kappa, u * W, &b0, &j0);
        plan_locate(P, batch, kappa, (u + 1) * W, &b1, &j1);
        const bool any = b0 < batch && (b0 != b1 || j0 != j1);
        int split = any ? u - (P[b0] + kappa) / W : 0;
        write_meta(meta + (size_t)u * kMetaInts, b0, j0, b1, j1, split, any ? seqlens[b0] : 0,
                   any ? splits[b0] + split : 0, any ? splits[b0 + 1] - splits[b0] : 0);
    }
    delete[] P;
}

hipError_t launch_plan(const int32_t* seqlens, int batch, int rows_wg, int num_units, int32_t* meta,
                       int32_t* splits, hipStream_t stream)
{
    size_t lds = sizeof(int) * (2 * (size_t)(batch + 1) + kPlanThreads / 64);
    if (batch <= 64) lds = sizeof(int) * 3 * 65 * (plan_threads(batch) / 64);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)plan_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(plan_threads(batch)), lds, stream, seqlens, batch, rows_wg,
                       num_units, meta, splits);
    return hipGetLastError();
}

}  // namespace mla
