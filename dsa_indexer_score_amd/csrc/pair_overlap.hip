// pair_overlap: adjacent-query top-k overlap diagnostic for gfx950.
//
// "Adjacent-Query KV-Index Overlap in 256K DSA Training" (sections 1 and 3)
// pairs queries without overlap, (q0,q1), (q2,q3), ..., and counts the exact
// intersection of their sorted KV-index rows by batched binary search rather
// than an all-pairs comparison.  One wave owns one pair: the partner row is
// staged into LDS (rows up to kStageMax entries; longer rows are searched in
// place), every lane binary-searches the partner for its own strided
// entries, and a wave reduction gives shared[i].
#include "kernels.h"

namespace dsai {
namespace {

constexpr int kWaves = 4;
constexpr int kStageMax = 4096;

__global__ void __launch_bounds__(kWaves * 64) pair_overlap_kernel(const int32_t *idx,
                                                                   const int32_t *valid_len,
                                                                   int64_t npairs, int W,
                                                                   int32_t *shared)
{
    __shared__ int32_t stage[kWaves][kStageMax];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t pr = (int64_t)blockIdx.x * kWaves + wave;
    if (pr >= npairs) return;  // no block-level barrier below
    const int32_t *a = idx + (2 * pr) * (int64_t)W;
    const int32_t *b = a + W;
    int va = valid_len[2 * pr], vb = valid_len[2 * pr + 1];
    va = va < 0 ? 0 : (va > W ? W : va);
    vb = vb < 0 ? 0 : (vb > W ? W : vb);
    const int32_t *bs = b;
    if (vb <= kStageMax) {
        for (int e = lane; e < vb; e += 64) stage[wave][e] = b[e];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        __builtin_amdgcn_wave_barrier();
        bs = stage[wave];
    }
    int c = 0;
    for (int e = lane; e < va; e += 64) {
        const int32_t x = a[e];
        int lo = 0, hi = vb;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (bs[mid] < x) lo = mid + 1;
            else hi = mid;
        }
        c += (lo < vb && bs[lo] == x) ? 1 : 0;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
    if (lane == 0) shared[pr] = c;
}

}  // namespace

hipError_t launch_pair_overlap(const int32_t *idx, const int32_t *valid_len, int64_t npairs,
                               int W, int32_t *shared, hipStream_t stream)
{
    if (npairs <= 0) return hipSuccess;
    const int64_t blocks = (npairs + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(pair_overlap_kernel, dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream,
                       idx, valid_len, npairs, W, shared);
    return hipGetLastError();
}

}  // namespace dsai
