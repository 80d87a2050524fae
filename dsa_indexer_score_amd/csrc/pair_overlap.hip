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
// entries are loaded once into registers (one memory round trip per pair),
// and window offsets are 32-bit (indices lie in [0, 2^31)), which keeps the
// wave at about 90 registers so five waves share each SIMD.
// Ranges wider than the bitmap are covered in consecutive windows.
// With few pairs (decode: a handful of rows spread over the whole context)
// one wave per pair would leave the chip idle and walk many small windows,
// so each pair gets a 1024-thread block and a 128 KB bitmap instead, which
// covers 2^20 positions per window (a 4M-token context in four).
// shared[i] counts the entries of row 2i present in row 2i+1.
#include "kernels.h"

namespace dsai {
namespace {

constexpr int kWaves = 4;
constexpr int kWords = 2048;                 // 8 KB of bitmap per wave
constexpr int64_t kWindow = (int64_t)kWords * 32;
constexpr int kRegPerLane = 36;              // rows up to 2304 entries stay in registers
constexpr int kUnroll = 8;                   // row entries in flight per lane (long rows)
constexpr int kRegionsUnroll = 32;           // region split: a 2048-entry row in one batch
constexpr int kWideThreads = 1024;           // few pairs: one block per pair ...
constexpr int kWideWords = 32768;            // ... with 128 KB of bitmap
constexpr int64_t kWideWindow = (int64_t)kWideWords * 32;
constexpr int64_t kWidePairsMax = 512;       // at most this many pairs take the block path

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

// f(x) for every entry x of row[0, n), U loads issued before use.
template <int U = kUnroll, class F>
__device__ __forceinline__ void for_each_index(const int32_t *row, int n, int lane, F &&f)
{
    for (int base = 0; base < n; base += 64 * U) {
        int32_t v[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int e = base + i * 64 + lane;
            v[i] = e < n ? row[e] : 0;
        }
#pragma unroll
        for (int i = 0; i < U; ++i)
            if (base + i * 64 + lane < n) f(v[i]);
    }
}

// f(valid, x) for every lane of every batch, in row order (entry base +
// 64 i + lane), kUnroll loads in flight; lanes past the row get valid = false
// so wave-uniform state in f stays uniform.
template <int U = kUnroll, class F>
__device__ __forceinline__ void for_each_index_ordered(const int32_t *row, int n, int lane, F &&f)
{
    for (int base = 0; base < n; base += 64 * U) {
        int32_t v[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int e = base + i * 64 + lane;
            v[i] = e < n ? row[e] : 0;
        }
#pragma unroll
        for (int i = 0; i < U; ++i) f(base + i * 64 + lane < n, v[i]);
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
        clear_words(bm, hi - lo + 1 < kWindow ? hi - lo + 1 : kWindow, lane);
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
                // entries and w0 lie in [0, 2^31): 32-bit offsets, and an
                // entry below the window wraps to >= 2^31
                const int32_t w0i = (int32_t)w0;
#pragma unroll
                for (int i = 0; i < kRegPerLane; ++i) {
                    const uint32_t r = (uint32_t)(rb[i] - w0i);
                    if (i * 64 + lane < vb && r < (uint32_t)kWindow)
                        atomicOr(&bm[r >> 5], 1u << (r & 31));
                }
                wave_sync_lds();
#pragma unroll
                for (int i = 0; i < kRegPerLane; ++i) {
                    const uint32_t r = (uint32_t)(ra[i] - w0i);
                    if (i * 64 + lane < va && r < (uint32_t)kWindow)
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

__global__ void __launch_bounds__(kWideThreads) pair_overlap_wide_kernel(
    const int32_t *idx, const int32_t *valid_len, int W, int32_t *shared)
{
    __shared__ __align__(16) uint32_t bm[kWideWords];
    __shared__ int red[kWideThreads / 64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t pr = blockIdx.x;
    const int32_t *a = idx + (2 * pr) * (int64_t)W;
    const int32_t *b = a + W;
    int va = valid_len[2 * pr], vb = valid_len[2 * pr + 1];
    va = va < 0 ? 0 : (va > W ? W : va);
    vb = vb < 0 ? 0 : (vb > W ? W : vb);
    int c = 0;
    if (va > 0 && vb > 0) {  // block-uniform
        const int64_t lo = a[0] < b[0] ? a[0] : b[0];
        const int64_t hi = a[va - 1] > b[vb - 1] ? a[va - 1] : b[vb - 1];
        for (int64_t w0 = lo; w0 <= hi; w0 += kWideWindow) {
            const int64_t nbits = hi - w0 + 1 < kWideWindow ? hi - w0 + 1 : kWideWindow;
            const int nq = (int)((nbits + 127) >> 7);  // 16-byte words of bitmap in use
            uint4 *bm4 = reinterpret_cast<uint4 *>(bm);
            for (int i = threadIdx.x; i < nq; i += kWideThreads) bm4[i] = make_uint4(0, 0, 0, 0);
            __syncthreads();
            for (int e = threadIdx.x; e < vb; e += kWideThreads) {
                const int64_t r = (int64_t)b[e] - w0;
                if (r >= 0 && r < nbits) atomicOr(&bm[r >> 5], 1u << (r & 31));
            }
            __syncthreads();
            for (int e = threadIdx.x; e < va; e += kWideThreads) {
                const int64_t r = (int64_t)a[e] - w0;
                if (r >= 0 && r < nbits) c += (bm[r >> 5] >> (r & 31)) & 1u;
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
    if (lane == 0) red[wave] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        int sum = 0;
#pragma unroll
        for (int i = 0; i < kWideThreads / 64; ++i) sum += red[i];
        shared[pr] = sum;
    }
}

// Three-region split of each pair (Overlap page, sections 6.1 and 6.4): the
// entries both rows hold, those only row 2i holds and those only row 2i+1
// holds, each ascending, written into fixed-capacity rows of width W (then
// -1) with the three counts.  Same bitmap windows as above, twice per
// window: row B's bits classify row A's entries, then row A's bits pick row
// B's unique entries.  Entries are visited in row order (e = 64 i + lane),
// so ballot-ranked appends keep every region sorted.  Rows of up to 2304
// entries are held in registers for all windows; longer rows are read
// again per pass.
__global__ void __launch_bounds__(kWaves * 64) pair_regions_kernel(
    const int32_t *idx, const int32_t *valid_len, int64_t npairs, int W, int32_t *shared,
    int32_t *left, int32_t *right, int32_t *counts)
{
    __shared__ uint32_t bitmap_all[kWaves][kWords];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t pr = (int64_t)blockIdx.x * kWaves + wave;
    if (pr >= npairs) return;  // no block-level barrier below
    uint32_t *bm = bitmap_all[wave];
    const int32_t *a = idx + (2 * pr) * (int64_t)W;
    const int32_t *b = a + W;
    int32_t *osh = shared + pr * (int64_t)W, *ol = left + pr * (int64_t)W,
            *orr = right + pr * (int64_t)W;
    int va = valid_len[2 * pr], vb = valid_len[2 * pr + 1];
    va = va < 0 ? 0 : (va > W ? W : va);
    vb = vb < 0 ? 0 : (vb > W ? W : vb);
    int nsh = 0, nl = 0, nr = 0;
    auto put = [&](int32_t *dst, int &n, bool take, int32_t x) {
        const uint64_t m = __ballot(take);
        if (take) dst[n + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = x;
        n += __popcll(m);
    };
    if ((va > 0 || vb > 0) && va <= 64 * kRegPerLane && vb <= 64 * kRegPerLane) {
        // both rows in registers (entry 64 i + lane in slot i): each row is
        // read from memory once, however many windows the pair's range needs
        const int64_t lo = va == 0 ? b[0] : (vb == 0 ? a[0] : (a[0] < b[0] ? a[0] : b[0]));
        const int64_t hi = va == 0 ? b[vb - 1]
                                   : (vb == 0 ? a[va - 1]
                                              : (a[va - 1] > b[vb - 1] ? a[va - 1] : b[vb - 1]));
        int32_t ra[kRegPerLane], rb[kRegPerLane];
#pragma unroll
        for (int i = 0; i < kRegPerLane; ++i) {
            const int e = i * 64 + lane;
            ra[i] = e < va ? a[e] : 0;
            rb[i] = e < vb ? b[e] : 0;
        }
        clear_words(bm, kWindow, lane);
        wave_sync_lds();
        for (int64_t w0 = lo; w0 <= hi; w0 += kWindow) {
            const int64_t nbits = hi - w0 + 1 < kWindow ? hi - w0 + 1 : kWindow;
            // entries and w0 lie in [0, 2^31): 32-bit offsets, and an entry
            // below the window wraps to >= 2^31
            const int32_t w0i = (int32_t)w0;
            // row B's bits; row A's entries -> shared or left-only
#pragma unroll
            for (int i = 0; i < kRegPerLane; ++i) {
                const uint32_t r = (uint32_t)(rb[i] - w0i);
                if (i * 64 + lane < vb && r < (uint32_t)kWindow) atomicOr(&bm[r >> 5], 1u << (r & 31));
            }
            wave_sync_lds();
#pragma unroll
            for (int i = 0; i < kRegPerLane; ++i) {
                if (i * 64 >= va) break;  // wave-uniform
                const uint32_t r = (uint32_t)(ra[i] - w0i);
                const bool in = i * 64 + lane < va && r < (uint32_t)kWindow;
                if (!__ballot(in)) continue;  // no entry of this slot in the window
                const bool hit = in && ((bm[r >> 5] >> (r & 31)) & 1u);
                put(osh, nsh, hit, ra[i]);
                put(ol, nl, in && !hit, ra[i]);
            }
            wave_sync_lds();
            clear_words(bm, nbits, lane);
            wave_sync_lds();
            // row A's bits; row B's entries -> right-only
#pragma unroll
            for (int i = 0; i < kRegPerLane; ++i) {
                const uint32_t r = (uint32_t)(ra[i] - w0i);
                if (i * 64 + lane < va && r < (uint32_t)kWindow) atomicOr(&bm[r >> 5], 1u << (r & 31));
            }
            wave_sync_lds();
#pragma unroll
            for (int i = 0; i < kRegPerLane; ++i) {
                if (i * 64 >= vb) break;  // wave-uniform
                const uint32_t r = (uint32_t)(rb[i] - w0i);
                const bool in = i * 64 + lane < vb && r < (uint32_t)kWindow;
                if (!__ballot(in)) continue;
                const bool hit = in && ((bm[r >> 5] >> (r & 31)) & 1u);
                put(orr, nr, in && !hit, rb[i]);
            }
            wave_sync_lds();
            clear_words(bm, nbits, lane);
            wave_sync_lds();
        }
    } else if (va > 0 || vb > 0) {
        const int64_t lo = va == 0 ? b[0] : (vb == 0 ? a[0] : (a[0] < b[0] ? a[0] : b[0]));
        const int64_t hi = va == 0 ? b[vb - 1]
                                   : (vb == 0 ? a[va - 1]
                                              : (a[va - 1] > b[vb - 1] ? a[va - 1] : b[vb - 1]));
        clear_words(bm, kWindow, lane);
        wave_sync_lds();
        for (int64_t w0 = lo; w0 <= hi; w0 += kWindow) {
            const int64_t nbits = hi - w0 + 1 < kWindow ? hi - w0 + 1 : kWindow;
            auto in_win = [&](int32_t x) { return (int64_t)x >= w0 && (int64_t)x - w0 < kWindow; };
            // row B's bits; row A's entries -> shared or left-only
            for_each_index<kRegionsUnroll>(b, vb, lane, [&](int32_t x) {
                if (in_win(x)) atomicOr(&bm[(x - w0) >> 5], 1u << ((x - w0) & 31));
            });
            wave_sync_lds();
            for_each_index_ordered<kRegionsUnroll>(a, va, lane, [&](bool valid, int32_t x) {
                const bool in = valid && in_win(x);
                const bool hit = in && ((bm[(x - w0) >> 5] >> ((x - w0) & 31)) & 1u);
                put(osh, nsh, hit, x);
                put(ol, nl, in && !hit, x);
            });
            wave_sync_lds();
            clear_words(bm, nbits, lane);
            wave_sync_lds();
            // row A's bits; row B's entries -> right-only
            for_each_index<kRegionsUnroll>(a, va, lane, [&](int32_t x) {
                if (in_win(x)) atomicOr(&bm[(x - w0) >> 5], 1u << ((x - w0) & 31));
            });
            wave_sync_lds();
            for_each_index_ordered<kRegionsUnroll>(b, vb, lane, [&](bool valid, int32_t x) {
                const bool in = valid && in_win(x);
                const bool hit = in && ((bm[(x - w0) >> 5] >> ((x - w0) & 31)) & 1u);
                put(orr, nr, in && !hit, x);
            });
            wave_sync_lds();
            clear_words(bm, nbits, lane);
            wave_sync_lds();
        }
    }
    for (int s = nsh + lane; s < W; s += 64) osh[s] = -1;
    for (int s = nl + lane; s < W; s += 64) ol[s] = -1;
    for (int s = nr + lane; s < W; s += 64) orr[s] = -1;
    if (lane == 0) {
        counts[3 * pr] = nsh;
        counts[3 * pr + 1] = nl;
        counts[3 * pr + 2] = nr;
    }
}

}  // namespace

hipError_t launch_pair_overlap(const int32_t *idx, const int32_t *valid_len, int64_t npairs,
                               int W, int32_t *shared, hipStream_t stream)
{
    if (npairs <= 0) return hipSuccess;
    if (npairs <= kWidePairsMax) {
        hipLaunchKernelGGL(pair_overlap_wide_kernel, dim3((unsigned)npairs), dim3(kWideThreads), 0,
                           stream, idx, valid_len, W, shared);
        return hipGetLastError();
    }
    const int64_t blocks = (npairs + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(pair_overlap_kernel, dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream,
                       idx, valid_len, npairs, W, shared);
    return hipGetLastError();
}

}  // namespace dsai

namespace dsai {

hipError_t launch_pair_regions(const int32_t *idx, const int32_t *valid_len, int64_t npairs, int W,
                               int32_t *shared, int32_t *left, int32_t *right, int32_t *counts,
                               hipStream_t stream)
{
    if (npairs <= 0) return hipSuccess;
    const int64_t blocks = (npairs + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(pair_regions_kernel, dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream,
                       idx, valid_len, npairs, W, shared, left, right, counts);
    return hipGetLastError();
}

}  // namespace dsai
