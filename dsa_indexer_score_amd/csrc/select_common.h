// Per-wave streaming top-k machinery shared by the streaming scoring kernel
// and the few-query selection kernels: order-preserving score codes, the packed LDS
// histogram, boundary searches, batched passes over a candidate list, exact
// radix cuts under the tie rule, and in-place compaction.
//
// A candidate list is a wave's buffer of (score bits, key) entries in
// ascending key order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsai {
namespace {

__device__ __forceinline__ uint32_t ord_code(uint32_t bits)
{
    if (bits == 0x80000000u) bits = 0;  // -0 -> +0
    return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

__device__ __forceinline__ int lane_rank(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive prefix sum over the 64 lanes (lane 0 first), in registers:
// Hillis-Steele steps within each 16-lane row, then the row totals.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x)
{
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

__device__ __forceinline__ uint32_t lane_value(uint32_t x, int l)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)x, l);
}

// Smallest float value whose order code is >= c: s >= code_floor_value(c)
// holds exactly when ord_code(s) >= c, for every finite s.
__device__ __forceinline__ float code_floor_value(uint32_t c)
{
    if (c >= 0x80000000u) return __uint_as_float(c & 0x7FFFFFFFu);
    if (c >= 0x007FFFFFu) return __uint_as_float(~c);
    return -__builtin_inff();
}

// Wait for this wave's outstanding LDS and global accesses.
__device__ __forceinline__ void wave_sync_mem()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
}

__host__ __device__ __forceinline__ int64_t visible_keys(int64_t pos, int64_t T, int m, int causal)
{
    if (!causal) return T;
    int64_t c = (pos + 1) / m;
    return c < T ? c : T;
}

// Key window of call row t in packed documents: the row's document doc (the
// largest with cu_q[doc] <= t; none for padding rows after cu_q[ndoc]), its
// position pos = pos0[doc] + t - cu_q[doc] inside the document, its visible
// keys [klo, klo + P) of the packed key array (the document's keys
// cu_k[doc] .. cu_k[doc + 1], clamped to [0, T)), and tok0 = cu_tok[doc], the
// packed token index of the document's position 0.  P = 0 for padding rows
// and negative positions.
struct DocWindow {
    int64_t pos = -1, P = 0, klo = 0, tok0 = 0;
};
template <class Params>
__device__ __forceinline__ DocWindow doc_window(const Params &p, int64_t t)
{
    DocWindow w;
    if (p.ndoc <= 0 || t < p.cu_q[0] || t >= p.cu_q[p.ndoc]) return w;
    int lo = 0, hi = p.ndoc;  // largest doc with cu_q[doc] <= t
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.cu_q[mid] <= t) lo = mid;
        else hi = mid;
    }
    const int doc = lo;
    w.pos = (p.pos0 ? p.pos0[doc] : 0) + (t - p.cu_q[doc]);
    const int64_t a = p.cu_k[doc], b = p.cu_k[doc + 1];
    w.klo = a < 0 ? 0 : (a > p.T ? p.T : a);
    const int64_t khi = b < w.klo ? w.klo : (b > p.T ? p.T : b);
    w.P = w.pos < 0 ? 0 : visible_keys(w.pos, khi - w.klo, p.m, p.causal);
    w.tok0 = p.cu_tok ? p.cu_tok[doc] : 0;
    return w;
}


// Few-query append (one wave, one row): the survivors of one batch of up to
// kFewBatch keys -- NG groups of 64, key0 + 64 g + lane in the row's local
// key order, sc[g] the lane's score, visible while below P -- whose order
// code is at least est.  They go to the candidate sub-list `cand` as one
// contiguous run in key order, reserved with one atomic on its count *cnt;
// the batch's directory entry records (offset, count).  Slots from `fewcap`
// on are counted but not stored (the row then goes to the repair launch).
template <int NG>
__device__ __forceinline__ void fq_append(const float (&sc)[NG], int64_t key0, int64_t P,
                                          uint32_t est, uint32_t *cnt, uint2 *cand,
                                          uint2 *dir_entry, int lane, int fewcap)
{
    uint64_t m[NG];
    uint32_t before[NG];
    uint32_t tot = 0;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const bool pass = key0 + 64 * g + lane < P && ord_code(__float_as_uint(sc[g])) >= est;
        m[g] = __ballot(pass);
        before[g] = tot;
        tot += (uint32_t)__popcll(m[g]);
    }
    uint32_t off = 0;
    if (tot) {
        if (lane == 0) off = atomicAdd(cnt, tot);
        off = (uint32_t)__builtin_amdgcn_readfirstlane((int)off);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const uint32_t i = off + before[g] + (uint32_t)lane_rank(m[g]);
            if (((m[g] >> lane) & 1ull) && i < (uint32_t)fewcap)
                cand[i] = make_uint2(__float_as_uint(sc[g]), (uint32_t)(key0 + 64 * g + lane));
        }
    }
    if (lane == 0) *dir_entry = make_uint2(off, tot);
}

// ---------------------------------------------------------------------------
// Selection helpers (one wave, one query).  Codes are cut in three radix
// levels: the top kB1 = 12 bits (the running histogram), then 10 and 10.
// `hist` holds kHistWords dwords of packed 16-bit counters (4096 bins); the
// 10-bit levels use the first 512 dwords.
// ---------------------------------------------------------------------------
constexpr int kB1 = 12;                         // bits of the running histogram
constexpr int kBins1 = 1 << kB1;
constexpr int kShift1 = 32 - kB1;               // bin of a code: u >> kShift1
constexpr int kHistWords = kBins1 / 2;

__device__ __forceinline__ void hist_clear(uint32_t *hist, int lane)
{
#pragma unroll
    for (int i = 0; i < kHistWords / 64; ++i) hist[lane + 64 * i] = 0;
}

__device__ __forceinline__ void hist_add(uint32_t *hist, uint32_t bin)
{
    atomicAdd(&hist[bin >> 1], 1u << ((bin & 1u) * 16));
}

__device__ __forceinline__ int hist_get(const uint32_t *hist, int bin)
{
    const uint32_t x = hist[bin >> 1];
    return (int)((bin & 1) ? (x >> 16) : (x & 0xFFFFu));
}

// Bin b with (count above b) < need <= (count above b) + h[b]; needs total >= need >= 1.
// Two lane-parallel levels: per-lane sums of nbins/64 bins with a suffix scan
// across lanes give the owning range, then one bin per lane inside it.
__device__ void find_boundary(const uint32_t *hist, int nbins, int need, int lane, int &b_out,
                              int &above_out, int &hb_out)
{
    const int per = nbins / 64, dpl = per / 2;
    // lane i sums range 63 - i of the bins, so a prefix over lanes is a
    // suffix over ranges (counted from the top bins down)
    const int ri = 63 - lane;
    uint32_t sum = 0;
    for (int i = 0; i < dpl; ++i) {
        uint32_t x = hist[ri * dpl + i];
        sum += (x & 0xFFFFu) + (x >> 16);
    }
    const uint32_t incl = wave_incl_scan(sum);
    const uint32_t excl = incl - sum;
    const uint64_t bm = __ballot(incl >= (uint32_t)need && excl < (uint32_t)need);
    int L0 = __ffsll((unsigned long long)bm) - 1;
    if (L0 < 0) L0 = 0;  // unreachable while the histogram matches the buffer
    const int owner = 63 - L0;
    const uint32_t base = lane_value(excl, L0);  // count above the owner's range
    // lane i < per takes bin owner*per + per-1-i (descending); inclusive prefix
    const int bin = owner * per + per - 1 - lane;
    const uint32_t h = lane < per ? (uint32_t)hist_get(hist, bin) : 0u;
    const uint32_t incl2 = wave_incl_scan(h);
    const uint64_t hit = __ballot(lane < per && base + incl2 >= (uint32_t)need);
    int L = __ffsll((unsigned long long)hit) - 1;
    if (L < 0) L = 0;
    b_out = owner * per + per - 1 - L;
    hb_out = (int)lane_value(h, L);
    above_out = (int)(base + lane_value(incl2, L) - (uint32_t)hb_out);
}

// Raise the running boundary bin tb (above = count in bins > tb) until
// above < need, 64 bins per step: lane i looks at bin tb + 1 + i, and the
// first lane whose inclusive prefix brings `above` below `need` is the new tb.
// Long runs of empty bins (e.g. all tiny magnitudes between -eps and +eps)
// cost one step per 64 bins.
__device__ void advance_boundary(const uint32_t *hist, int need, int lane, int &tb, int &above)
{
    while (above >= need) {
        const int b = tb + 1 + lane;
        const int incl = (int)wave_incl_scan(b < kBins1 ? (uint32_t)hist_get(hist, b) : 0u);
        const uint64_t ok = __ballot(above - incl < need);
        if (ok) {
            const int L = __ffsll((unsigned long long)ok) - 1;
            tb += 1 + L;
            above -= (int)lane_value((uint32_t)incl, L);
            return;
        }
        tb += 64;
        above -= (int)lane_value((uint32_t)incl, 63);
    }
}

// Visit buf[0, cnt) in buffer order, kBatch chunks of 64 entries at a time:
// all loads of a batch are issued before any of them is consumed, so a pass
// costs a few memory round trips per 512 entries instead of one per 64.  The
// callback may store into buf at or below the entry it was given (in-place
// compaction): later batches are read before those positions are reached.
constexpr int kBatch = 8;
template <class F>
__device__ __forceinline__ void for_each_entry(const uint2 *buf, int cnt, int lane, F &&f)
{
    for (int base = 0; base < cnt; base += 64 * kBatch) {
        uint2 v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int e = base + i * 64 + lane;
            v[i] = e < cnt ? buf[e] : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) f(base + i * 64 + lane < cnt, v[i]);
    }
}

struct Cut {
    uint32_t tc;  // keep u >= tc (exact == 0) or u > tc plus the first need_eq of u == tc
    int exact;
    int need_eq;
};

// Levels 2 and 3 of the radix cut: `src(f)` feeds every candidate code of the
// level-1 boundary bin b1 to f (from the buffer or from an LDS gather), a1 is
// the count above b1.  Returns the cut that keeps exactly `need` entries.
template <class Src>
__device__ Cut refine_cut(Src &&src, int need, int b1, int a1, uint32_t *hist, int lane)
{
    Cut c;
    wave_sync_mem();
    hist_clear(hist, lane);
    wave_sync_mem();
    src([&](uint32_t u) { hist_add(hist, (u >> 10) & 1023u); });
    wave_sync_mem();
    int b2, a2, h2;
    find_boundary(hist, 1024, need - a1, lane, b2, a2, h2);
    const int above = a1 + a2;
    const uint32_t pre = ((uint32_t)b1 << 10) | (uint32_t)b2;  // top 22 bits
    if (above + h2 == need) {
        c.tc = pre << 10;
        c.exact = 0;
        c.need_eq = 0;
        return c;
    }
    wave_sync_mem();
    hist_clear(hist, lane);
    wave_sync_mem();
    src([&](uint32_t u) {
        if ((u >> 10) == pre) hist_add(hist, u & 1023u);
    });
    wave_sync_mem();
    int b3, a3, h3;
    find_boundary(hist, 1024, need - above, lane, b3, a3, h3);
    c.tc = (pre << 10) | (uint32_t)b3;
    c.exact = 1;
    c.need_eq = need - above - a3;
    return c;
}

// Cut that keeps at least `need` of the buffer's best entries.  With
// allow_approx, a level-1 bin edge is accepted when it keeps at most
// `approx_limit` entries; otherwise the cut is exact (keeps exactly `need`).
__device__ Cut choose_cut(const uint2 *buf, int cnt, int need, uint32_t *hist, bool allow_approx,
                          int approx_limit, int lane)
{
    int b1, a1, h1;
    find_boundary(hist, kBins1, need, lane, b1, a1, h1);
    if ((allow_approx && a1 + h1 <= approx_limit) || a1 + h1 == need) {
        Cut c;
        c.tc = (uint32_t)b1 << kShift1;
        c.exact = 0;
        c.need_eq = 0;
        return c;
    }
    auto src = [&](auto &&f) {
        for_each_entry(buf, cnt, lane, [&](bool valid, uint2 v) {
            const uint32_t u = ord_code(v.x);
            if (valid && (u >> kShift1) == (uint32_t)b1) f(u);
        });
    };
    return refine_cut(src, need, b1, a1, hist, lane);
}

// Exact cut for the final selection: the codes of the level-1 boundary bin
// are gathered (one batched pass, buffer order) into `gather` (LDS, gcap
// entries) and refined there; a bin larger than gcap refines from the buffer.
__device__ Cut final_cut(const uint2 *buf, int cnt, int need, uint32_t *hist, uint32_t *gather,
                         int gcap, int lane)
{
    int b1, a1, h1;
    find_boundary(hist, kBins1, need, lane, b1, a1, h1);
    if (a1 + h1 == need || h1 > gcap) return choose_cut(buf, cnt, need, hist, false, 0, lane);
    int gcnt = 0;
    for_each_entry(buf, cnt, lane, [&](bool valid, uint2 v) {
        const uint32_t u = ord_code(v.x);
        const bool in = valid && (u >> kShift1) == (uint32_t)b1;
        const uint64_t m = __ballot(in);
        if (in) gather[gcnt + lane_rank(m)] = u;
        gcnt += __popcll(m);
    });
    auto src = [&](auto &&f) {
        for (int i = lane; i < gcnt; i += 64) f(gather[i]);
    };
    return refine_cut(src, need, b1, a1, hist, lane);
}

// Stable in-place compaction of buf[0, cnt) under `cut`; rebuilds the histogram.
__device__ void compact(uint2 *buf, int &cnt, const Cut &cut, uint32_t *hist, int lane)
{
    wave_sync_mem();
    hist_clear(hist, lane);
    wave_sync_mem();
    int wcnt = 0, eqseen = 0;
    for_each_entry(buf, cnt, lane, [&](bool valid, uint2 v) {
        const uint32_t u = ord_code(v.x);
        bool keep;
        if (cut.exact) {
            const bool eq = valid && u == cut.tc;
            const uint64_t em = __ballot(eq);
            keep = valid && (u > cut.tc || (eq && eqseen + lane_rank(em) < cut.need_eq));
            eqseen += __popcll(em);
        } else {
            keep = valid && u >= cut.tc;
        }
        const uint64_t km = __ballot(keep);
        if (keep) {
            buf[wcnt + lane_rank(km)] = v;
            hist_add(hist, u >> kShift1);
        }
        wcnt += __popcll(km);
    });
    cnt = wcnt;
    wave_sync_mem();
}

}  // namespace
}  // namespace dsai
