// select_dense: exact top-k of a few queries' materialised scores.
//
// For a handful of query rows (decode, small batches against a long key
// set) the scoring kernel runs in its dense mode (one or two rows: the rows
// kernel of score_rows.hip) and writes each row's visible scores to the
// workspace (a [rows, T] array: kilobytes to tens of
// megabytes here, never the prefill-sized tensor).  Three kernels then find
// the same exact result as the streaming selection -- the Ksel best keys
// under the total order (higher score first, equal scores to the lower key
// index, DoSA summary, "Prerequisites") written in ascending key order
// ("Adjacent-Query KV-Index Overlap in 256K DSA Training", section 3),
// expanded and followed by the tail (GLM-5.3-Flash Module 06 "DSA & KPool",
// section 2):
//  1. candidates: per row, a sample (128 blocks of 64 keys) gives an
//     estimated threshold a little below the expected Ksel-th score
//     (estimate_kernel); per (row, 4096-key segment), every key at or above
//     it is kept in key order (filter_kernel, all CUs); per row, the
//     segments are concatenated in order into an LDS list (finish_kernel).
//     The true selection is contained in that list whenever the list holds
//     at least Ksel keys (all of them are >= the estimate, so the Ksel-th
//     best is too); otherwise -- or if the list would overflow, e.g. under
//     massive ties -- the steps below run over the full row instead;
//  2. exact cut: a 4096-bin histogram of the order codes' top 12 bits gives
//     the bin holding the Ksel-th code; if that bin does not end the
//     selection exactly, two more 10-bit histograms over the codes of that
//     bin give the exact Ksel-th code c and how many entries equal to c are
//     kept;
//  3. ordered output: a block-wide prefix count of entries above c and of
//     entries equal to c (packed into one 32-bit scan) gives each kept key
//     its output slot, so ties go to the lowest keys.
// Passes over the row read chunks of 16K keys (the filter: segments of 4K),
// 16 consecutive keys per thread loaded as four 16-byte vectors, so each
// thread has its loads in flight together; histograms use LDS atomics only.
#include "kernels.h"
#include "select_common.h"

namespace dsai {
namespace {

constexpr int kDenseThreads = 1024;
constexpr int kDenseWaves = kDenseThreads / 64;
constexpr int kPer = 16;                        // consecutive keys per thread per chunk
constexpr int kChunk = kDenseThreads * kPer;    // keys per chunk
constexpr int kFilterThreads = 256;             // candidate filter block
constexpr int kSeg = kFilterThreads * kPer;     // keys per filter segment
constexpr int64_t kFilterBlocks = 4096;         // filter blocks per launch (about)

// The KP consecutive scores of this thread's slice of chunk `base` (raw
// bits); all loads are issued before any is used.
template <int KP>
struct SliceT {
    uint32_t bits[KP];
    __device__ void load(const uint32_t *sc, int base, int n)
    {
        const int j0 = base + (int)threadIdx.x * KP;
        if (j0 + KP <= n) {
            const uint4 *v = reinterpret_cast<const uint4 *>(sc + j0);
#pragma unroll
            for (int i = 0; i < KP / 4; ++i) {
                const uint4 x = v[i];
                bits[4 * i] = x.x;
                bits[4 * i + 1] = x.y;
                bits[4 * i + 2] = x.z;
                bits[4 * i + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < KP; ++i) bits[i] = j0 + i < n ? sc[j0 + i] : 0u;
        }
    }
};
using Slice = SliceT<kPer>;

// Exclusive prefix sum over the block's NW waves of threads (thread order)
// and its total.
template <int NW = kDenseWaves>
__device__ uint32_t block_excl_scan(uint32_t x, uint32_t *red, uint32_t &total)
{
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
// hist[b], for 1 <= need <= total.  Thread i owns nbins/1024 consecutive bins
// counted down from the top, so a prefix over threads is a suffix over bins.
__device__ void block_boundary(const uint32_t *hist, int nbins, uint32_t need, uint32_t *red,
                               uint32_t *res, int &b, uint32_t &above, uint32_t &hb)
{
    const int per = nbins / kDenseThreads;
    const int top = nbins - 1 - (int)threadIdx.x * per;
    uint32_t s = 0;
    for (int i = 0; i < per; ++i) s += hist[top - i];
    uint32_t tot;
    const uint32_t ex = block_excl_scan(s, red, tot);
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
// prefix bin holding the need-th code (a lower bound, exact = false).
template <int LEVELS = 3, class Src>
__device__ void block_exact_cut(Src &&src, uint32_t need, uint32_t *hist, uint32_t *red,
                                uint32_t *res, uint32_t &tc, bool &exact, uint32_t &need_eq)
{
    exact = false;
    need_eq = 0;
    for (int i = threadIdx.x; i < kBins1; i += kDenseThreads) hist[i] = 0;
    __syncthreads();
    src([&](uint32_t u) { atomicAdd(&hist[u >> kShift1], 1u); });
    __syncthreads();
    int b1;
    uint32_t a1, h1;
    block_boundary(hist, kBins1, need, red, res, b1, a1, h1);
    if (a1 + h1 == need) {
        tc = (uint32_t)b1 << kShift1;
        return;
    }
    for (int i = threadIdx.x; i < 1024; i += kDenseThreads) hist[i] = 0;
    __syncthreads();
    src([&](uint32_t u) {
        if ((u >> kShift1) == (uint32_t)b1) atomicAdd(&hist[(u >> 10) & 1023u], 1u);
    });
    __syncthreads();
    int b2;
    uint32_t a2, h2;
    block_boundary(hist, 1024, need - a1, red, res, b2, a2, h2);
    const uint32_t pre = ((uint32_t)b1 << 10) | (uint32_t)b2;  // top 22 bits
    const uint32_t above = a1 + a2;
    if (LEVELS == 2 || above + h2 == need) {
        tc = pre << 10;
        return;
    }
    for (int i = threadIdx.x; i < 1024; i += kDenseThreads) hist[i] = 0;
    __syncthreads();
    src([&](uint32_t u) {
        if ((u >> 10) == pre) atomicAdd(&hist[u & 1023u], 1u);
    });
    __syncthreads();
    int b3;
    uint32_t a3, h3;
    block_boundary(hist, 1024, need - above, red, res, b3, a3, h3);
    tc = (pre << 10) | (uint32_t)b3;
    exact = true;
    need_eq = need - above - a3;
}

// Output slots of one thread's consecutive entries under a cut: counts of
// entries above / equal to the cut before this thread (block-wide, plus the
// running totals of earlier rounds), then each kept entry's slot in order.
struct CutCounter {
    uint32_t tc, need_eq;
    bool exact;
    uint32_t gt_run = 0, eq_run = 0;
    __device__ bool gt(bool valid, uint32_t u) const { return valid && (exact ? u > tc : u >= tc); }
    __device__ bool eq(bool valid, uint32_t u) const { return valid && exact && u == tc; }
    __device__ uint32_t kept() const { return gt_run + (eq_run < need_eq ? eq_run : need_eq); }
};

constexpr int kCap = 8192;            // candidate list (LDS), also the sample size
constexpr int kSampleBlock = 64;      // consecutive keys per sample block
constexpr uint32_t kAllKeys = 0u;     // estimate: every key is a candidate
constexpr uint32_t kNoList = 0xFFFFFFFFu;  // estimate: select from the full row

// One row of the dense scores: score j is key klo + j; an output key j is
// written as klo + j, or expanded as tok0 + j m + x (packed documents: the
// row's document window and token offset; else klo = tok0 = 0).
struct RowView {
    int64_t t, pos, P, klo, tok0;
    int n;
    const uint32_t *sc;
    uint32_t need;
    __device__ RowView(const ScoreSelectParams &p, int64_t qrow)
    {
        t = p.row0 + qrow;
        if (p.varlen) {
            const DocWindow w = doc_window(p, t);
            pos = w.pos;
            P = w.P < p.sstride ? w.P : p.sstride;  // at most the dense row
            klo = w.klo;
            tok0 = w.tok0;
        } else {
            pos = p.q_pos0 + t;
            P = visible_keys(pos, p.T, p.m, p.causal);
            klo = tok0 = 0;
        }
        n = (int)P;
        sc = reinterpret_cast<const uint32_t *>(p.scores + qrow * p.sstride);
        need = (uint32_t)(n < p.ksel ? n : p.ksel);
    }
};

// Threshold estimate of each row: the c-th best code of a sample of 128
// blocks of 64 keys spread over the row (to a 22-bit prefix: the lower edge
// of the prefix bin holding it), c about 1.5x the sample's expected share of
// the selection plus a margin, so that the keys at or above it almost always
// hold the whole selection and fit the candidate list.
__global__ void __launch_bounds__(kDenseThreads) estimate_kernel(ScoreSelectParams p)
{
    __shared__ uint32_t hist[kBins1];
    __shared__ uint32_t sample[kCap];
    __shared__ uint32_t red[kDenseWaves];
    __shared__ uint32_t res[3];
    const RowView rv(p, blockIdx.x);
    uint32_t est = kAllKeys;
    if (rv.n > kCap) {
        const uint32_t c =
            (uint32_t)((3ull * rv.need * kCap) / (2ull * (uint64_t)rv.n)) + 8u;
        est = kNoList;
        if (c <= (uint32_t)kCap) {
            const int spacing = (rv.n - kSampleBlock) / (kCap / kSampleBlock - 1);
            for (int s = threadIdx.x; s < kCap; s += kDenseThreads)
                sample[s] = ord_code(rv.sc[(s / kSampleBlock) * spacing + s % kSampleBlock]);
            __syncthreads();
            uint32_t est_eq;
            bool est_exact;
            block_exact_cut<2>(  // a lower bound of the c-th code is all it needs
                [&](auto &&f) {
                    for (int i = threadIdx.x; i < kCap; i += kDenseThreads) f(sample[i]);
                },
                c, hist, red, res, est, est_exact, est_eq);  // low bits 0: never kNoList
        }
    }
    if (threadIdx.x == 0) p.est[blockIdx.x] = est;
}

// Candidates of one row, segment by segment (kSeg keys each): every visible
// key whose code is >= the row's estimate, as (score bits, key) in key
// order, into the segment's slot, and the segment's count.  A block takes
// every gridDim.x-th segment of its row that holds visible keys, so the
// grid does not grow with the rows' stride (packed documents: a row's
// window is often a small part of all keys).  Without an estimate the cut
// reads the full row and no count is needed.
__global__ void __launch_bounds__(kFilterThreads) filter_kernel(ScoreSelectParams p)
{
    __shared__ uint32_t red[kFilterThreads / 64];
    const RowView rv(p, blockIdx.y);
    const uint32_t est = p.est[blockIdx.y];
    if (est == kNoList) return;
    for (int seg = blockIdx.x; (int64_t)seg * kSeg < rv.n; seg += gridDim.x) {
        const int base = seg * kSeg;
        const int64_t slot = (int64_t)blockIdx.y * p.nseg + seg;
        Slice sl;
        sl.load(rv.sc, base, rv.n);
        const int j0 = base + (int)threadIdx.x * kPer;
        uint32_t cnt = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            cnt += (j0 + i < rv.n && ord_code(sl.bits[i]) >= est) ? 1u : 0u;
        uint32_t tot;
        uint32_t o = block_excl_scan<kFilterThreads / 64>(cnt, red, tot);  // ends in a barrier
        uint2 *dst = p.seg_buf + slot * (int64_t)kSeg;
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (j0 + i < rv.n && ord_code(sl.bits[i]) >= est)
                dst[o++] = make_uint2(sl.bits[i], (uint32_t)(j0 + i));
        if (threadIdx.x == 0) p.seg_cnt[slot] = (int32_t)tot;
    }
}

// Exact selection of one row and its canonical output row: from the
// candidate list (segments concatenated in key order) when it holds the
// selection and fits in LDS, else from the full row.
__global__ void __launch_bounds__(kDenseThreads) finish_kernel(ScoreSelectParams p)
{
    __shared__ uint32_t hist[kBins1];
    __shared__ uint32_t cbits[kCap];  // candidates' raw score bits
    __shared__ int32_t ckey[kCap];
    __shared__ uint32_t soff[kDenseThreads];
    __shared__ uint16_t owner[kCap];
    __shared__ uint32_t red[kDenseWaves];
    __shared__ uint32_t res[3];

    const int64_t qrow = blockIdx.x;
    const RowView rv(p, qrow);
    const int64_t t = rv.t, pos = rv.pos, P = rv.P;
    const int n = rv.n;
    const uint32_t *sc = rv.sc;
    const uint32_t need = rv.need;
    const int mexp = p.expand ? p.m : 1;
    const int64_t obase = p.expand ? rv.tok0 : rv.klo;  // output of key j: obase + j mexp + x
    int32_t *orow = p.idx + t * (int64_t)p.W;
    float *srow = p.sel_score ? p.sel_score + t * (int64_t)p.W : nullptr;

    auto row_src = [&](auto &&f) {  // every visible score of the row, from memory
        for (int base = 0; base < n; base += kChunk) {
            Slice sl;
            sl.load(sc, base, n);
            const int j0 = base + (int)threadIdx.x * kPer;
#pragma unroll
            for (int i = 0; i < kPer; ++i)
                if (j0 + i < n) f(ord_code(sl.bits[i]));
        }
    };

    // ---- the segments' candidates, concatenated in key order.  The first
    // round's counts are loaded together with the estimate.
    int ncand = -1;  // -1: the list is not usable, select from the full row
    const int nseg_row = (n + kSeg - 1) / kSeg;
    const int32_t *cnts = p.seg_cnt + qrow * (int64_t)p.nseg;
    const uint32_t est = p.est[qrow];
    const uint32_t c_first =
        (int)threadIdx.x < nseg_row ? (uint32_t)cnts[threadIdx.x] : 0u;
    if (est != kNoList) {
        const uint2 *cands = p.seg_buf + qrow * (int64_t)p.nseg * kSeg;
        uint32_t total = 0, off_first = 0, tot_first = 0;
        for (int s0 = 0; s0 < nseg_row; s0 += kDenseThreads) {
            const int sg = s0 + (int)threadIdx.x;
            const uint32_t c = s0 == 0 ? c_first : (sg < nseg_row ? (uint32_t)cnts[sg] : 0u);
            uint32_t tot;
            const uint32_t off = block_excl_scan(c, red, tot);
            if (s0 == 0) {
                off_first = off;
                tot_first = tot;
            }
            total += tot;
        }
        if (total >= need && total <= (uint32_t)kCap) {
            ncand = (int)total;
            const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
            uint32_t done = 0;
            for (int s0 = 0; s0 < nseg_row; s0 += kDenseThreads) {
                const int sg = s0 + (int)threadIdx.x;
                uint32_t off = off_first, tot = tot_first;
                if (s0 > 0)
                    off = block_excl_scan(sg < nseg_row ? (uint32_t)cnts[sg] : 0u, red, tot);
                soff[threadIdx.x] = done + off;
                __syncthreads();
                // owner segment of each list slot of this round (LDS only) ...
                const int nr = nseg_row - s0 < kDenseThreads ? nseg_row - s0 : kDenseThreads;
                for (int r = wave; r < nr; r += kDenseWaves) {
                    const uint32_t o = soff[r];
                    const uint32_t end = r + 1 < nr ? soff[r + 1] : done + tot;
                    for (uint32_t i = o + lane; i < end; i += 64) owner[i] = (uint16_t)r;
                }
                __syncthreads();
                // ... then one slot per thread and step, every load independent
                constexpr int kSlots = kCap / kDenseThreads;
                uint2 cv[kSlots];
#pragma unroll
                for (int x = 0; x < kSlots; ++x) {
                    const uint32_t i = done + threadIdx.x + (uint32_t)x * kDenseThreads;
                    cv[x] = make_uint2(0u, 0u);
                    if (i < done + tot) {
                        const int r = owner[i];
                        cv[x] = cands[(int64_t)(s0 + r) * kSeg + (i - soff[r])];
                    }
                }
#pragma unroll
                for (int x = 0; x < kSlots; ++x) {
                    const uint32_t i = done + threadIdx.x + (uint32_t)x * kDenseThreads;
                    if (i < done + tot) {
                        cbits[i] = cv[x].x;
                        ckey[i] = (int32_t)cv[x].y;
                    }
                }
                __syncthreads();
                done += tot;
            }
        }
    }

    CutCounter cc;
    cc.tc = 0;
    cc.exact = false;
    cc.need_eq = 0;
    if (ncand >= 0) {
        // ---- exact selection within the list, then its ordered output
        if ((uint32_t)ncand > need)
            block_exact_cut(
                [&](auto &&f) {
                    for (int i = threadIdx.x; i < ncand; i += kDenseThreads) f(ord_code(cbits[i]));
                },
                need, hist, red, res, cc.tc, cc.exact, cc.need_eq);
        constexpr int kPerC = kCap / kDenseThreads;
        const int i0 = (int)threadIdx.x * kPerC;
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int i = 0; i < kPerC; ++i) {
            const bool valid = i0 + i < ncand;
            const uint32_t u = valid ? ord_code(cbits[i0 + i]) : 0u;
            ngt += cc.gt(valid, u) ? 1u : 0u;
            neq += cc.eq(valid, u) ? 1u : 0u;
        }
        uint32_t tot;
        const uint32_t ex = block_excl_scan(ngt | (neq << 16), red, tot);
        uint32_t gt_before = ex & 0xFFFFu, eq_before = ex >> 16;
#pragma unroll
        for (int i = 0; i < kPerC; ++i) {
            const bool valid = i0 + i < ncand;
            const uint32_t bits = valid ? cbits[i0 + i] : 0u;
            const uint32_t u = valid ? ord_code(bits) : 0u;
            const bool gt = cc.gt(valid, u), eq = cc.eq(valid, u);
            if (gt || (eq && eq_before < cc.need_eq)) {
                const uint32_t kb = gt_before + (eq_before < cc.need_eq ? eq_before : cc.need_eq);
                const int key = ckey[i0 + i];
                for (int x = 0; x < mexp; ++x) {
                    orow[(int)kb * mexp + x] = (int32_t)(obase + (int64_t)key * mexp + x);
                    if (srow) srow[(int)kb * mexp + x] = __uint_as_float(bits);
                }
            }
            gt_before += gt ? 1u : 0u;
            eq_before += eq ? 1u : 0u;
        }
        cc.gt_run = tot & 0xFFFFu;
        cc.eq_run = tot >> 16;
    } else {
        // ---- fallback: radix passes and the ordered output over the full row
        if ((uint32_t)n > need) block_exact_cut(row_src, need, hist, red, res, cc.tc, cc.exact,
                                                cc.need_eq);
        for (int base = 0; base < n; base += kChunk) {
            Slice sl;
            sl.load(sc, base, n);
            const int j0 = base + (int)threadIdx.x * kPer;
            uint32_t ngt = 0, neq = 0;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const uint32_t u = ord_code(sl.bits[i]);
                ngt += cc.gt(j0 + i < n, u) ? 1u : 0u;
                neq += cc.eq(j0 + i < n, u) ? 1u : 0u;
            }
            uint32_t tot;
            const uint32_t ex = block_excl_scan(ngt | (neq << 16), red, tot);
            uint32_t gt_before = cc.gt_run + (ex & 0xFFFFu);
            uint32_t eq_before = cc.eq_run + (ex >> 16);
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const uint32_t u = ord_code(sl.bits[i]);
                const bool gt = cc.gt(j0 + i < n, u), eq = cc.eq(j0 + i < n, u);
                if (gt || (eq && eq_before < cc.need_eq)) {
                    const uint32_t kb =
                        gt_before + (eq_before < cc.need_eq ? eq_before : cc.need_eq);
                    for (int x = 0; x < mexp; ++x) {
                        orow[(int)kb * mexp + x] = (int32_t)(obase + (int64_t)(j0 + i) * mexp + x);
                        if (srow) srow[(int)kb * mexp + x] = __uint_as_float(sl.bits[i]);
                    }
                }
                gt_before += gt ? 1u : 0u;
                eq_before += eq ? 1u : 0u;
            }
            cc.gt_run += tot & 0xFFFFu;
            cc.eq_run += tot >> 16;
        }
    }

    const int body = (int)cc.kept() * mexp;
    int tl = (p.expand && p.tail && p.causal) ? (int)(pos + 1 - P * p.m) : 0;
    tl = tl < 0 ? 0 : (tl > p.W - body ? p.W - body : tl);  // packed documents: keys missing
    for (int s = body + (int)threadIdx.x; s < p.W; s += kDenseThreads) {
        orow[s] = s < body + tl ? (int32_t)(rv.tok0 + P * p.m + (s - body)) : -1;
        if (srow) srow[s] = 0.f;
    }
    if (threadIdx.x == 0) p.valid_len[t] = body + tl;
}

}  // namespace

hipError_t launch_select_dense(const ScoreSelectParams &p, hipStream_t stream)
{
    if (p.nrows <= 0) return hipSuccess;
    hipLaunchKernelGGL(estimate_kernel, dim3((unsigned)p.nrows), dim3(kDenseThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // about 16 filter blocks per CU, at most one per segment of the stride
    const int64_t per_row = (kFilterBlocks + p.nrows - 1) / p.nrows;
    const int64_t fx = per_row < p.nseg ? per_row : p.nseg;
    hipLaunchKernelGGL(filter_kernel, dim3((unsigned)fx, (unsigned)p.nrows),
                       dim3(kFilterThreads), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(finish_kernel, dim3((unsigned)p.nrows), dim3(kDenseThreads), 0, stream, p);
    return hipGetLastError();
}

int dense_segment_keys() { return kSeg; }

}  // namespace dsai
