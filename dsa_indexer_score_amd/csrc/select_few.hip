// select_few: exact top-k of the few-query path's candidates (decode, small
// batches against a long key set).
//
// The few-query path never writes a score array.  The scoring launches
// (score_rows.hip, or the streaming kernel in its few-query mode) first
// score a sample of each row's keys; estimate_kernel cuts a threshold from
// it; the second scoring launch keeps only the keys whose scores reach it,
// appended per batch of kFewBatch keys to the row's candidate list with a
// directory entry (offset, count) per batch (the DoSA summary's sparse
// write-back, "Method steps").  finish_kernel then finds the same exact
// result as the streaming selection -- the Ksel best keys under the total
// order (higher score first, equal scores to the lower key index, DoSA
// summary, "Prerequisites") written in ascending key order ("Adjacent-Query
// KV-Index Overlap in 256K DSA Training", section 3), expanded and followed
// by the tail (GLM-5.3-Flash Module 06 "DSA & KPool", section 2):
//  1. candidates: the batches' runs (each in the sub-list its batch index
//     picks) are concatenated in batch order, which is key order, into an
//     LDS list.  The list holds the selection whenever
//     it has at least Ksel entries (all of them are >= the estimate, so the
//     Ksel-th best is too).  Otherwise -- too high an estimate, or more
//     candidates than the list or a sub-list holds (massive ties,
//     adversarial orders) --
//     the row is marked for the repair launch, the streaming kernel run on
//     the marked rows only;
//  2. exact cut: a 4096-bin histogram of the order codes' top 12 bits gives
//     the bin holding the Ksel-th code; if that bin does not end the
//     selection exactly, two more 10-bit histograms over the codes of that
//     bin give the exact Ksel-th code c and how many entries equal to c are
//     kept;
//  3. ordered output: a block-wide prefix count of entries above c and of
//     entries equal to c (packed into one 32-bit scan) gives each kept key
//     its output slot, so ties go to the lowest keys.
#include "block_cut.h"
#include "kernels.h"
#include "select_common.h"

namespace dsai {
namespace {

constexpr int kDenseThreads = 1024;
constexpr int kDenseWaves = kDenseThreads / 64;

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

constexpr int kCap = kFewCap;         // candidate list (LDS)
constexpr int kSampleBlock = 64;      // consecutive keys per sample place
static_assert(kSampleKeys % kSampleBlock == 0 && kCap % kDenseThreads == 0, "layout");

// One few-query row: its visible keys are local keys 0 .. n-1 (key klo + j
// of the key array); an output key j is written as klo + j, or expanded as
// tok0 + j m + x (packed documents: the row's document window and token
// offset; else klo = tok0 = 0).
struct RowView {
    int64_t t, pos, P, klo, tok0;
    int64_t n;
    uint32_t need;
    __device__ RowView(const ScoreSelectParams &p, int64_t qrow)
    {
        t = p.row0 + qrow;
        if (p.varlen) {
            const DocWindow w = doc_window(p, t);
            pos = w.pos;
            P = w.P < p.row_keys ? w.P : p.row_keys;  // at most a row's directory
            klo = w.klo;
            tok0 = w.tok0;
        } else {
            pos = p.q_pos0 + t;
            P = visible_keys(pos, p.T, p.m, p.causal);
            klo = tok0 = 0;
        }
        n = P;
        need = (uint32_t)(n < p.ksel ? n : p.ksel);
    }
};

// Threshold estimate of each row (sample_estimate), when the filtering
// launch does not compute it itself.  With witness keys (DoSA summary,
// "Method steps": decode takes keys selected at an earlier step as
// witnesses), the need-th best of their exact scores is a lower bound of
// the row's need-th best score -- any need visible keys bound it from below
// -- so the estimate is raised to it when it is higher: the keys at or
// above it then hold the selection whenever the witnesses name need
// distinct visible keys.  (Repeated keys can make it too high; the cut then
// finds fewer candidates than it needs and the row goes to the repair
// launch, as for any failed estimate.)  Also zeroes the row's candidate
// counts for the filtering launch that follows.
__global__ void __launch_bounds__(kDenseThreads) estimate_kernel(ScoreSelectParams p)
{
    __shared__ uint32_t hist[kBins1];
    __shared__ uint32_t sample[kSampleKeys];
    __shared__ uint32_t red[kDenseWaves];
    __shared__ uint32_t res[3];
    const RowView rv(p, blockIdx.x);
    if (threadIdx.x < kFewSub) p.fq_cnt[blockIdx.x * kFewSub + threadIdx.x] = 0;
    const float *sm = p.samp + (int64_t)blockIdx.x * kSampStride;
    if (rv.n > kCap) {
        for (int s = threadIdx.x; s < kSampleKeys; s += kDenseThreads)
            sample[s] = ord_code(__float_as_uint(sm[s]));
        __syncthreads();
    }
    uint32_t est = sample_estimate<kDenseThreads>(
        [&](auto &&f) {
            for (int i = threadIdx.x; i < kSampleKeys; i += kDenseThreads) f(sample[i]);
        },
        rv.n, rv.need, hist, red, res);
    const int nw = p.witness && !p.varlen ? (p.nwit < kWitnessMax ? p.nwit : kWitnessMax) : 0;
    if (rv.n > kCap && nw > 0) {
        // the witness scores (entries naming no visible key hold -inf)
        const uint32_t none = ord_code(__float_as_uint(-__builtin_inff()));
        __syncthreads();
        uint32_t nvalid = 0;
        for (int s = threadIdx.x; s < nw; s += kDenseThreads) {
            const uint32_t u = ord_code(__float_as_uint(sm[kSampleKeys + s]));
            sample[s] = u;
            nvalid += u != none ? 1u : 0u;
        }
        uint32_t tot;
        block_excl_scan<kDenseThreads>(nvalid, red, tot);
        if (tot >= rv.need) {
            uint32_t tw, tw_eq;
            bool tw_exact;
            block_exact_cut<kDenseThreads, 3, true>(  // the need-th witness code itself
                [&](auto &&f) {
                    for (int i = threadIdx.x; i < nw; i += kDenseThreads) f(sample[i]);
                },
                rv.need, hist, red, res, tw, tw_exact, tw_eq);
            if (est == kNoList || tw > est) est = tw;
        }
    }
    if (threadIdx.x == 0) p.est[blockIdx.x] = est;
}

// Exact selection of one row from its candidate list and its canonical
// output row; a row whose list cannot hold the selection is marked for the
// repair launch (status 1) and left to it.
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
    const uint32_t need = rv.need;
    // the first directory round, the sub-lists' counts and the estimate are
    // loaded together; then the counts' total, and whether one overflowed
    const int nbat = (int)((rv.n + kFewBatch - 1) / kFewBatch);
    const uint2 *dir = p.fq_dir + qrow * p.nbatch;
    const uint2 de_first = (int)threadIdx.x < nbat ? dir[threadIdx.x] : make_uint2(0u, 0u);
    const uint32_t est = p.est[qrow];
    if (threadIdx.x < 64) {
        const uint32_t c = threadIdx.x < kFewSub ? p.fq_cnt[qrow * kFewSub + threadIdx.x] : 0u;
        uint32_t tot = c;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off);
        const bool over = __ballot(c > (uint32_t)kFewSubCap) != 0ull;
        if (threadIdx.x == 0) {
            res[0] = tot;
            res[1] = over;
        }
    }
    __syncthreads();
    const uint32_t total = res[0];
    if (est == kNoList || res[1] || total < need || total > (uint32_t)kCap) {
        if (threadIdx.x == 0) p.status[qrow] = 1;
        return;
    }
    if (threadIdx.x == 0) p.status[qrow] = 0;
    const int ncand = (int)total;
    const int mexp = p.expand ? p.m : 1;
    const int64_t obase = p.expand ? rv.tok0 : rv.klo;  // output of key j: obase + j mexp + x
    int32_t *orow = p.idx + t * (int64_t)p.W;
    float *srow = p.sel_score ? p.sel_score + t * (int64_t)p.W : nullptr;

    // ---- the batches' runs, concatenated in batch (= key) order: thread i
    // of a round owns batch s0 + i
    {
        const uint2 *cands = p.ws + qrow * (int64_t)p.cap;
        uint32_t done = 0;
        for (int s0 = 0; s0 < nbat; s0 += kDenseThreads) {
            const int sg = s0 + (int)threadIdx.x;
            const uint2 de = s0 == 0 ? de_first
                                     : (sg < nbat ? dir[sg] : make_uint2(0u, 0u));  // (offset, count)
            const uint32_t at = (uint32_t)(sg % kFewSub) * kFewSubCap + de.x;  // run start
            uint32_t tot;
            const uint32_t off = block_excl_scan<kDenseThreads>(de.y, red, tot);
            // the list slots of the batch's run name it as their owner, and
            // the batch records the shift from list slot to buffer position
            for (uint32_t i = 0; i < de.y; ++i) owner[done + off + i] = (uint16_t)threadIdx.x;
            soff[threadIdx.x] = at - (done + off);
            __syncthreads();
            // one slot per thread and step, every load independent
            constexpr int kSlots = kCap / kDenseThreads;
            uint2 cv[kSlots];
#pragma unroll
            for (int x = 0; x < kSlots; ++x) {
                const uint32_t i = done + threadIdx.x + (uint32_t)x * kDenseThreads;
                cv[x] = make_uint2(0u, 0u);
                if (i < done + tot) cv[x] = cands[i + soff[owner[i]]];
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

    // ---- exact selection within the list, then its ordered output
    CutCounter cc;
    cc.tc = 0;
    cc.exact = false;
    cc.need_eq = 0;
    if ((uint32_t)ncand > need)
        block_exact_cut<kDenseThreads>(
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
    const uint32_t ex = block_excl_scan<kDenseThreads>(ngt | (neq << 16), red, tot);
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

hipError_t launch_few_estimate(const ScoreSelectParams &p, hipStream_t stream)
{
    if (p.nrows <= 0) return hipSuccess;
    hipLaunchKernelGGL(estimate_kernel, dim3((unsigned)p.nrows), dim3(kDenseThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_few_finish(const ScoreSelectParams &p, hipStream_t stream)
{
    if (p.nrows <= 0) return hipSuccess;
    hipLaunchKernelGGL(finish_kernel, dim3((unsigned)p.nrows), dim3(kDenseThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace dsai
