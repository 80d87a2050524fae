// Block-wide radix cuts over 32-bit order codes (gfx950), shared by the
// few-query path's estimate, its exact cut and the rows kernel: a 4096-bin
// histogram of the codes' top 12 bits, then 10-bit histograms of the bin
// that holds the cut, so the need-th best code is found in up to three
// passes over the codes with no sort.  NT is the block's thread count (a
// multiple of 64 that divides 1024).
#pragma once
#include "kernels.h"
#include "select_common.h"

namespace dsai {
namespace {

constexpr uint32_t kAllKeys = 0u;          // estimate: every key is a candidate
constexpr uint32_t kNoList = 0xFFFFFFFFu;  // estimate: leave the row to the repair launch

// Exclusive prefix sum over the block's NT threads (thread order) and its
// total; red holds NT / 64 words.
template <int NT>
__device__ uint32_t block_excl_scan(uint32_t x, uint32_t *red, uint32_t &total)
{
    constexpr int NW = NT / 64;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint32_t incl = wave_incl_scan(x);
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint32_t v = red[i];
        off += i < wave ? v : 0u;
        tot += v;
    }
    __syncthreads();
    total = tot;
    return off + incl - x;
}

// Bin b of hist[0, nbins) with (count above b) < need <= (count above b) +
// hist[b], for 1 <= need <= total.  Thread i owns nbins/NT consecutive bins
// counted down from the top, so a prefix over threads is a suffix over bins.
template <int NT>
__device__ void block_boundary(const uint32_t *hist, int nbins, uint32_t need, uint32_t *red,
                               uint32_t *res, int &b, uint32_t &above, uint32_t &hb)
{
    const int per = nbins / NT;
    const int top = nbins - 1 - (int)threadIdx.x * per;
    uint32_t s = 0;
    for (int i = 0; i < per; ++i) s += hist[top - i];
    uint32_t tot;
    const uint32_t ex = block_excl_scan<NT>(s, red, tot);
    if (ex < need && ex + s >= need) {  // exactly one thread
        uint32_t acc = ex;
        for (int i = 0; i < per; ++i) {
            const uint32_t h = hist[top - i];
            if (acc + h >= need) {
                res[0] = (uint32_t)(top - i);
                res[1] = acc;
                res[2] = h;
                break;
            }
            acc += h;
        }
    }
    __syncthreads();
    b = (int)res[0];
    above = res[1];
    hb = res[2];
    __syncthreads();
}

// Exact cut keeping `need` of the codes that src(f) feeds to f (each thread
// feeds its own share): keep codes > tc plus the first need_eq codes equal
// to tc in key order (exact), or every code >= tc.  1 <= need <= count.
// LEVELS = 2 stops after the 22-bit prefix: tc is then the lower edge of the
// prefix bin holding the need-th code (a lower bound, exact = false).  FULL:
// no early stop where a bin edge already separates the need best codes; tc
// is then always the need-th code itself.
template <int NT, int LEVELS = 3, bool FULL = false, class Src>
__device__ void block_exact_cut(Src &&src, uint32_t need, uint32_t *hist, uint32_t *red,
                                uint32_t *res, uint32_t &tc, bool &exact, uint32_t &need_eq)
{
    exact = false;
    need_eq = 0;
    for (int i = threadIdx.x; i < kBins1; i += NT) hist[i] = 0;
    __syncthreads();
    src([&](uint32_t u) { atomicAdd(&hist[u >> kShift1], 1u); });
    __syncthreads();
    int b1;
    uint32_t a1, h1;
    block_boundary<NT>(hist, kBins1, need, red, res, b1, a1, h1);
    if (!FULL && a1 + h1 == need) {
        tc = (uint32_t)b1 << kShift1;
        return;
    }
    for (int i = threadIdx.x; i < 1024; i += NT) hist[i] = 0;
    __syncthreads();
    src([&](uint32_t u) {
        if ((u >> kShift1) == (uint32_t)b1) atomicAdd(&hist[(u >> 10) & 1023u], 1u);
    });
    __syncthreads();
    int b2;
    uint32_t a2, h2;
    block_boundary<NT>(hist, 1024, need - a1, red, res, b2, a2, h2);
    const uint32_t pre = ((uint32_t)b1 << 10) | (uint32_t)b2;  // top 22 bits
    const uint32_t above = a1 + a2;
    if (LEVELS == 2 || (!FULL && above + h2 == need)) {
        tc = pre << 10;
        return;
    }
    for (int i = threadIdx.x; i < 1024; i += NT) hist[i] = 0;
    __syncthreads();
    src([&](uint32_t u) {
        if ((u >> 10) == pre) atomicAdd(&hist[u & 1023u], 1u);
    });
    __syncthreads();
    int b3;
    uint32_t a3, h3;
    block_boundary<NT>(hist, 1024, need - above, red, res, b3, a3, h3);
    tc = (pre << 10) | (uint32_t)b3;
    exact = true;
    need_eq = need - above - a3;
}


// Threshold estimate of a few-query row from its sample (kSampleKeys exact
// scores at samp, the row's n visible keys, need = min(n, Ksel)): kAllKeys
// when every key fits the candidate list, else the c-th best code of the
// sample to a 22-bit prefix (the lower edge of the prefix bin holding it),
// c about 1.5x the sample's expected share of the selection plus a margin,
// so that the keys at or above it almost always hold the whole selection
// and fit the list; kNoList when c exceeds the sample.  Block-wide (all NT
// threads); the same value for any NT.
template <int NT, class Src>
__device__ uint32_t sample_estimate(Src &&src, int64_t n, uint32_t need, uint32_t *hist,
                                    uint32_t *red, uint32_t *res)
{
    if (n <= kFewCap) return kAllKeys;
    const uint64_t c = (3ull * need * kSampleKeys) / (2ull * (uint64_t)n) + 8u;
    if (c > (uint64_t)kSampleKeys) return kNoList;
    uint32_t est, est_eq;
    bool est_exact;
    block_exact_cut<NT, 2>(src, (uint32_t)c, hist, red, res, est, est_exact, est_eq);
    return est;  // low bits 0: never kNoList
}

}  // namespace
}  // namespace dsai
