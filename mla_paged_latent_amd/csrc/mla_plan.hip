// Split-KV tile plan for variable-length decode batches.
//
// The pages state only that the decode kernel is tuned for serving sequences
// of varying length (GeekNews release note, id.news.hada.io; FlashMLA
// explainer section 2.4 on padding waste). The plan below is this library's
// own: every cache block of the batch sits at a position on a cost line
// (sequence b starts at P[b] and pays a fixed segment cost kappa before its
// first block), and unit u takes the blocks whose position falls in
// [u*W, (u+1)*W) with W = ceil(total / num_units). Every block therefore
// belongs to exactly one unit, each unit's blocks are contiguous in
// (sequence, block) order, and no unit costs more than W + kappa.
//
// The device planner (one workgroup) and the host planner evaluate the same
// integer formulas from mla_common.h, so their outputs agree bit for bit.
#include "mla_common.h"

namespace mla {

constexpr int kPlanThreads = 1024;

// Inclusive prefix sum of a[0..n) in LDS by one workgroup of kPlanThreads.
__device__ void block_inclusive_scan(int* a, int n, int* carry)
{
    const int tid = threadIdx.x;
    const int per = (n + kPlanThreads - 1) / kPlanThreads;
    const int lo = tid * per;
    const int hi = min(lo + per, n);
    int local = 0;
    for (int k = lo; k < hi; ++k) local += a[k];
    carry[tid] = local;
    __syncthreads();
    // Hillis-Steele over the per-thread sums
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        int v = (tid >= off) ? carry[tid - off] : 0;
        __syncthreads();
        carry[tid] += v;
        __syncthreads();
    }
    int run = carry[tid] - local;        // exclusive offset of this thread's chunk
    for (int k = lo; k < hi; ++k) {
        run += a[k];
        a[k] = run;
    }
    __syncthreads();
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ seqlens, int batch,
                                                             int kappa, int num_units,
                                                             int32_t* __restrict__ meta,
                                                             int32_t* __restrict__ splits)
{
    extern __shared__ int plan_smem[];
    int* P = plan_smem;                  // [batch + 1]
    int* NS = P + (batch + 1);           // [batch + 1]
    int* carry = NS + (batch + 1);       // [kPlanThreads]
    const int tid = threadIdx.x;

    for (int b = tid; b < batch; b += kPlanThreads) {
        int nb = blocks_of(seqlens[b]);
        P[b + 1] = nb > 0 ? nb + kappa : 0;
    }
    if (tid == 0) P[0] = 0;
    __syncthreads();
    block_inclusive_scan(P + 1, batch, carry);

    const int W = plan_width(P[batch], num_units);
    for (int b = tid; b < batch; b += kPlanThreads) {
        int cost = P[b + 1] - P[b];
        int nb = cost > 0 ? cost - kappa : 0;
        NS[b + 1] = plan_splits(P[b], nb, kappa, W);
    }
    if (tid == 0) NS[0] = 0;
    __syncthreads();
    block_inclusive_scan(NS + 1, batch, carry);
    for (int b = tid; b <= batch; b += kPlanThreads) splits[b] = NS[b];

    for (int u = tid; u < num_units; u += kPlanThreads) {
        int b0, j0, b1, j1;
        plan_locate(P, batch, kappa, u * W, &b0, &j0);
        plan_locate(P, batch, kappa, (u + 1) * W, &b1, &j1);
        int split = (b0 < batch && (b0 != b1 || j0 != j1)) ? u - (P[b0] + kappa) / W : 0;
        int32_t* m = meta + (size_t)u * kMetaInts;
        m[0] = b0; m[1] = j0; m[2] = b1; m[3] = j1; m[4] = split;
        m[5] = 0; m[6] = 0; m[7] = 0;
    }
}

void plan_host(const int32_t* seqlens, int batch, int kappa, int num_units, int32_t* meta, int32_t* splits)
{
    int* P = new int[batch + 1];
    P[0] = 0;
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
        int split = (b0 < batch && (b0 != b1 || j0 != j1)) ? u - (P[b0] + kappa) / W : 0;
        int32_t* m = meta + (size_t)u * kMetaInts;
        m[0] = b0; m[1] = j0; m[2] = b1; m[3] = j1; m[4] = split;
        m[5] = 0; m[6] = 0; m[7] = 0;
    }
    delete[] P;
}

hipError_t launch_plan(const int32_t* seqlens, int batch, int kappa, int num_units, int32_t* meta,
                       int32_t* splits, hipStream_t stream)
{
    size_t lds = sizeof(int) * (2 * (size_t)(batch + 1) + kPlanThreads);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)plan_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), lds, stream, seqlens, batch, kappa,
                       num_units, meta, splits);
    return hipGetLastError();
}

}  // namespace mla
