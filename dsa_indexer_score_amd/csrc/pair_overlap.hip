// pair_overlap: adjacent-query top-k overlap diagnostic for gfx950.
//
// "Adjacent-Query KV-Index Overlap in 256K DSA Training" (sections 1 and 3)
// pairs queries without overlap, (q0,q1), (q2,q3), ..., and counts the exact
// intersection of their sorted KV-index rows without an all-pairs
// comparison.  One wave owns one pair and a bitmap in LDS over the pair's
// index range [lo, hi] (lo = smallest first entry, hi = largest last entry
// of the two ascending rows): the wave sets one bit per entry of row B,
// tests the bit of every entry of row A, then zeroes the words it used.
// Every LDS access is independent of the others, so the wave is bound by
// loading the two rows, not by the latency of a search; rows of up to 2304
// entries are loaded once into registers (one memory round trip per pair).
// Ranges wider than the bitmap are covered in consecutive windows.
// shared[i] counts the entries of row 2i present in row 2i+1.
#include "kernels.h"

namespace dsai {
namespace {

constexpr int kWaves = 4;
constexpr int kWords = 2048;                 // 8 KB of bitmap per wave
constexpr int64_t kWindow = (int64_t)kWords * 32;
constexpr int kRegPerLane = 36;              // rows up to 2304 entries stay in registers
constexpr int kUnroll = 8;                   // row entries in flight per lane (long rows)

__device__ __forceinline__ void wave_sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ void clear_words(uint32_t *bm, int64_t nbits, int lane)
{
    const int nw = (int)((nbits + 31) >> 5);
    for (int i = lane; i < nw; i += 64) bm[i] = 0;
}

// f(x) for every entry x of row[0, n), kUnroll loads issued before use.
template <class F>
__device__ __forceinline__ void for_each_index(const int32_t *row, int n, int lane, F &&f)
{
    for (int base = 0; base < n; base += 64 * kUnroll) {
        int32_t v[kUnroll];
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const int e = base + i * 64 + lane;
            v[i] = e < n ? row[e] : 0;
        }
#pragma unroll
        for (int i = 0; i < kUnroll; ++i)
            if (base + i * 64 + lane < n) f(v[i]);
    }
}

__global__ void __launch_bounds__(kWaves * 64) pair_overlap_kernel(const int32_t *idx,
                                                                   const int32_t *valid_len,
                                                                   int64_t npairs, int W,
                                                                   int32_t *shared)
{
    __shared__ uint32_t bitmap_all[kWaves][kWords];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t pr = (int64_t)blockIdx.x * kWaves + wave;
    if (pr >= npairs) return;  // no block-level barrier below
    uint32_t *bm = bitmap_all[wave];
    const int32_t *a = idx + (2 * pr) * (int64_t)W;
    const int32_t *b = a + W;
    int va = valid_len[2 * pr], vb = valid_len[2 * pr + 1];
    va = va < 0 ? 0 : (va > W ? W : va);
    vb = vb < 0 ? 0 : (vb > W ? W : vb);
    int c = 0;
    if (va > 0 && vb > 0) {
        const int64_t lo = a[0] < b[0] ? a[0] : b[0];
        const int64_t hi = a[va - 1] > b[vb - 1] ? a[va - 1] : b[vb - 1];
        clear_words(bm, kWindow, lane);
        wave_sync_lds();
        if (va <= 64 * kRegPerLane && vb <= 64 * kRegPerLane) {
            // both rows in registers: one round trip to memory per pair
            int32_t ra[kRegPerLane], rb[kRegPerLane];
#pragma unroll
            for (int i = 0; i < kRegPerLane; ++i) {
                const int e = i * 64 + lane;
                ra[i] = e < va ? a[e] : 0;
                rb[i] = e < vb ? b[e] : 0;
            }
            for (int64_t w0 = lo; w0 <= hi; w0 += kWindow) {
#pragma unroll
                for (int i = 0; i < kRegPerLane; ++i) {
                    const int64_t r = (int64_t)rb[i] - w0;
                    if (i * 64 + lane < vb && r >= 0 && r < kWindow)
                        atomicOr(&bm[r >> 5], 1u << (r & 31));
                }
                wave_sync_lds();
#pragma unroll
                for (int i = 0; i < kRegPerLane; ++i) {
                    const int64_t r = (int64_t)ra[i] - w0;
                    if (i * 64 + lane < va && r >= 0 && r < kWindow)
                        c += (bm[r >> 5] >> (r & 31)) & 1u;
                }
                wave_sync_lds();
                clear_words(bm, hi - w0 + 1 < kWindow ? hi - w0 + 1 : kWindow, lane);
                wave_sync_lds();
            }
        } else {
            for (int64_t w0 = lo; w0 <= hi; w0 += kWindow) {
                for_each_index(b, vb, lane, [&](int32_t x) {
                    const int64_t r = (int64_t)x - w0;
                    if (r >= 0 && r < kWindow) atomicOr(&bm[r >> 5], 1u << (r & 31));
                });
                wave_sync_lds();
                for_each_index(a, va, lane, [&](int32_t x) {
                    const int64_t r = (int64_t)x - w0;
                    if (r >= 0 && r < kWindow) c += (bm[r >> 5] >> (r & 31)) & 1u;
                });
                wave_sync_lds();
                clear_words(bm, hi - w0 + 1 < kWindow ? hi - w0 + 1 : kWindow, lane);
                wave_sync_lds();
            }
        }
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
