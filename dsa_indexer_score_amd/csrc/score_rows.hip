// score_rows: few-query scoring (decode, small batches, batched decode over
// packed documents) for gfx950.
//
// Computes, for the keys j visible to row t,
//     s_tj = sum_h w[t,h] * ReLU(q[t,h,:] . k[j,:])
// (DoSA: Dots Sparse Attention, summary page, "Prerequisites") in one of two
// modes:
//  * sample: the exact scores of a fixed sample of the row's keys (64
//    consecutive keys in each of kSampleKeys / 64 places spread over the
//    row), from which the row's threshold estimate is cut, and of the row's
//    witness keys when the caller gives them (keys of an earlier selection,
//    whose exact scores bound the threshold from below: DoSA summary,
//    "Method steps", decode);
//  * filter: every visible key, keeping only the (score, key) pairs at or
//    above the row's estimate -- appended to the row's candidate list one
//    run of kFewBatch keys at a time, with the run's directory entry -- so no
//    score array is ever written (the DoSA summary's sparse write-back: only
//    scores that reach the threshold leave the registers).
// The dot products use the same MFMA operands and instruction order as the
// fused streaming kernel, and the signed-ReLU head sum the same fma order
// (head block by head block, accumulator element by element, then the two
// lane halves, then k_scale), so every score is bit-identical to the one the
// streaming selection sees.
//
// Why a kernel of its own: the streaming kernel's block shares each LDS key
// tile among 8 waves that hold 8 different rows; with one row, 7 of them idle
// and each block walks its key range through barriers.  Here every wave holds
// the rows' q operands in registers and owns a run of 64-key groups of one
// row slab; it loads its keys' B operands straight from global memory (each
// lane the contiguous half of one key row that its MFMA slots cover, so 32
// keys arrive as whole rows), one or two groups ahead, with no LDS and no
// barrier.
// All CUs stream disjoint slices of the key set, so one row is bound by
// reading the keys from HBM.  Slabs of the same key range sit in blocks a
// multiple of 8 apart, so they land on the same XCD and share its L2.
#include "kernels.h"
#include "mfma_ops.h"
#include "select_common.h"

namespace dsai {
namespace {

constexpr int kRowsWaves = 4;
constexpr int kRowsThreads = kRowsWaves * 64;
// waves per launch, each streaming several groups: about one per SIMD, two
// for packed documents (many rows, each a slab of its own)
constexpr int kTargetWaves = 1024;
constexpr int kTargetWavesDocs = 2048;

constexpr int kBatchGroups = kFewBatch / kSelGroup;     // groups per candidate run
constexpr int kSampleGroups = kSampleKeys / kSelGroup;  // groups per row sample

// Witness entries scored per row, and the key that entry i of row t names
// (-1: none, or not visible to the row, which sees keys 0 .. P-1).
__device__ __host__ inline int64_t witness_count(const ScoreSelectParams &p)
{
    return p.witness ? (p.nwit < kWitnessMax ? p.nwit : kWitnessMax) : 0;
}
__device__ inline int64_t witness_key(const ScoreSelectParams &p, int64_t t, int64_t i, int64_t P)
{
    if (i >= witness_count(p)) return -1;
    const int32_t e = p.witness[t * p.wit_stride + i];
    if (e < 0 || (p.expand && e % p.m)) return -1;
    const int64_t key = p.expand ? e / p.m : e;
    return key < P ? key : -1;
}

template <int DT, int NB, int D, int SQ, bool VARLEN, bool SAMPLE>
__global__ void __launch_bounds__(kRowsThreads) score_rows_kernel(ScoreSelectParams p)
{
    static_assert(!VARLEN || SQ == 1, "packed documents: one row per slab");
    static_assert(!SAMPLE || SQ == 1, "samples: one row per slab");
    using O = Op<DT, D>;
    using A = typename O::A;
    constexpr int KS = O::KS, ES = O::ES, RAW = O::RAW;
    constexpr bool kScaled = DT >= 2;  // fp8 codes: per-row scales fold out of the ReLU
    constexpr int64_t ROWB = (int64_t)D * ES;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int hh = lane >> 5, l32 = lane & 31;

    // rows of this slab and the keys they see: keys [klo, klo + Pq[i]) of
    // the key array (klo = 0 but for packed documents, one row per slab)
    const int64_t r0 = (int64_t)blockIdx.y * SQ;
    int64_t Pq[SQ];
    int64_t Pmax = 0, klo = 0;
#pragma unroll
    for (int i = 0; i < SQ; ++i) {
        const int64_t r = r0 + i;
        if constexpr (VARLEN) {
            // a window longer than a row's directory (the caller's bound on a
            // document's keys) is cut to it: every store stays in the row
            const DocWindow dw = r < p.nrows ? doc_window(p, p.row0 + r) : DocWindow{};
            Pq[i] = dw.P < p.row_keys ? dw.P : p.row_keys;
            klo = dw.klo;
        } else {
            Pq[i] = r < p.nrows ? visible_keys(p.q_pos0 + p.row0 + r, p.T, p.m, p.causal) : 0;
        }
        Pmax = Pq[i] > Pmax ? Pq[i] : Pmax;
    }
    // sample: rows of at most kFewCap keys need no estimate (all their keys
    // are candidates); group g starts at key g * spacing
    int64_t spacing = kSelGroup;
    if constexpr (SAMPLE) {
        if (Pmax <= kFewCap) return;
        spacing = (Pmax - kSelGroup) / (kSampleGroups - 1);
    }
    // the slab's 64-key groups (sample: then the witness groups), split
    // evenly over the slab's waves in runs of whole candidate batches
    const int64_t nwg = SAMPLE && !VARLEN ? (witness_count(p) + kSelGroup - 1) / kSelGroup : 0;
    const int64_t ngroups = SAMPLE ? kSampleGroups + nwg : (Pmax + kSelGroup - 1) / kSelGroup;
    const int64_t nwaves = (int64_t)gridDim.x * kRowsWaves;
    int64_t gpw = (ngroups + nwaves - 1) / nwaves;
    if (!SAMPLE) gpw = (gpw + kBatchGroups - 1) / kBatchGroups * kBatchGroups;
    const int64_t g0 = ((int64_t)blockIdx.x * kRowsWaves + wave) * gpw;
    if (g0 >= ngroups) return;
    const int64_t g1 = g0 + gpw < ngroups ? g0 + gpw : ngroups;

    // q operands and folded head weights of the slab's rows.  Every load is
    // issued unconditionally from a clamped, valid address and masked
    // afterwards, so the loads are in flight together instead of one
    // branch (and one wait) each.
    A qa[SQ][NB][KS];
    float wv[SQ][NB][16];
    const char *qbytes = static_cast<const char *>(p.q);
#pragma unroll
    for (int i = 0; i < SQ; ++i) {
        const bool active = r0 + i < p.nrows;
        const int64_t t = p.row0 + (active ? r0 + i : 0);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int head = 32 * b + l32;
            const bool okq = active && head < p.H;
            O::load_a(qbytes + ((t * p.H + (okq ? head : 0)) * (int64_t)D) * ES, hh, qa[i][b]);
            if (!okq) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) qa[i][b][ks] = O::zero();
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int h2 = 32 * b + 8 * (v >> 2) + 4 * hh + (v & 3);
                const bool ok = active && h2 < p.H;
                const int hc = ok ? h2 : 0;
                float wt = p.w[t * p.w_stride + hc];
                if (kScaled) wt *= p.q_scale[t * p.H + hc];
                wv[i][b][v] = ok ? wt : 0.f;
            }
        }
    }

    // B operands of one 64-key group: column block c holds keys 64g + 32c + l32.
    // A key at or past T is read at key T - 1 instead: column j of the
    // product depends on key j alone, and such keys' scores are never stored.
    const char *kbytes = static_cast<const char *>(p.k);
    // groups loaded ahead of use: two where the register budget allows
    // (fp8 at d = 128: 16 KB of keys per wave in flight), else one
    constexpr int AHEAD = RAW <= 4 ? 2 : 1;
    uint4 raw[AHEAD + 1][2][RAW];
    float ksc[AHEAD + 1] = {};
    // witness group g (>= kSampleGroups): entries 64 (g - kSampleGroups) + j
    const int64_t trow = p.row0 + r0;  // the slab's row (one in sample mode)
    auto key_of = [&](int64_t g, int j) -> int64_t {
        if (SAMPLE && g >= kSampleGroups) {
            const int64_t key = witness_key(p, trow, (g - kSampleGroups) * kSelGroup + j, Pq[0]);
            return key < 0 ? 0 : key;
        }
        const int64_t key = klo + g * spacing + j;
        return key < p.T ? key : p.T - 1;
    };
    auto load_group = [&](int64_t g, uint4 (&dst)[2][RAW], float &sc) {
#pragma unroll
        for (int c = 0; c < 2; ++c) raw_row<O, D>(kbytes + key_of(g, 32 * c + l32) * ROWB, hh, dst[c]);
        if (kScaled) sc = p.k_scale[key_of(g, lane)];
    };
    // filter: the rows' estimates, and the scores of the current batch
    uint32_t est[SQ];
    float bsc[SQ][kBatchGroups];
#pragma unroll
    for (int i = 0; i < SQ; ++i) {
        est[i] = SAMPLE || r0 + i >= p.nrows ? 0u : p.est[r0 + i];
#pragma unroll
        for (int x = 0; x < kBatchGroups; ++x) bsc[i][x] = 0.f;
    }

#pragma unroll
    for (int a = 0; a < AHEAD; ++a)
        if (g0 + a < g1) load_group(g0 + a, raw[a], ksc[a]);
    for (int64_t g = g0; g < g1; ++g) {
        if (g + AHEAD < g1) load_group(g + AHEAD, raw[AHEAD], ksc[AHEAD]);
        float part[SQ][2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            A bfr[KS];
            O::from_raw(raw[0][c], bfr);
#pragma unroll
            for (int i = 0; i < SQ; ++i) {
                float e = 0.f;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    f32x16 acc;
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) acc = O::mma(qa[i][b][ks], bfr[ks], acc);
#pragma unroll
                    for (int v = 0; v < 16; ++v) e = fmaf(wv[i][b][v], fmaxf(acc[v], 0.f), e);
                }
                part[i][c] = e;
            }
        }
        const int gb = (int)(g % kBatchGroups);  // group within its candidate batch
#pragma unroll
        for (int i = 0; i < SQ; ++i) {
            // lanes < 32 own keys 0..31 of the group, lanes >= 32 keys 32..63:
            // each adds the two 16-head halves of its key's sum
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[i][0]),
                                                             __float_as_uint(part[i][1]), false,
                                                             false);
            float s = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            if (kScaled) s *= ksc[0];
            if constexpr (SAMPLE) {
                // witness entries that name no visible key rank below every score
                if (g >= kSampleGroups &&
                    witness_key(p, trow, (g - kSampleGroups) * kSelGroup + lane, Pq[0]) < 0)
                    s = -__builtin_inff();
                p.samp[(r0 + i) * kSampStride + g * kSelGroup + lane] = s;
            } else {
#pragma unroll
                for (int x = 0; x < kBatchGroups; ++x)
                    if (x == gb) bsc[i][x] = s;
            }
        }
        // the batch is complete: its survivors go to the rows' candidate lists
        if (!SAMPLE && (gb == kBatchGroups - 1 || g + 1 == g1)) {
            const int64_t b = g / kBatchGroups;
#pragma unroll
            for (int i = 0; i < SQ; ++i) {
                const int64_t r = r0 + i;
                if (r >= p.nrows) continue;
                // a batch ends early only where the slab's keys end (runs are
                // whole batches): its groups past g are masked off here
                float sc[kBatchGroups];
#pragma unroll
                for (int x = 0; x < kBatchGroups; ++x) sc[x] = x <= gb ? bsc[i][x] : 0.f;
                const int64_t kend = b * kFewBatch + (gb + 1) * (int64_t)kSelGroup;
                const int sub = (int)(b % kFewSub);
                fq_append<kBatchGroups>(sc, b * kFewBatch, Pq[i] < kend ? Pq[i] : kend, est[i],
                                        p.fq_cnt + r * kFewSub + sub,
                                        p.ws + r * (int64_t)p.cap + sub * kFewSubCap,
                                        p.fq_dir + r * p.nbatch + b, lane, kFewSubCap);
            }
        }
        if (g + 1 < g1) {
#pragma unroll
            for (int a = 0; a < AHEAD; ++a) {
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int x = 0; x < RAW; ++x) raw[a][c][x] = raw[a + 1][c][x];
                ksc[a] = ksc[a + 1];
            }
        }
    }
}

template <int DT, int NB, int D, int SQ, bool VARLEN, bool SAMPLE>
hipError_t launch_rows(const ScoreSelectParams &p, hipStream_t stream)
{
    // the last row sees the most keys (packed documents: at most row_keys)
    const int64_t pmax =
        VARLEN ? p.row_keys : visible_keys(p.q_pos0 + p.row0 + p.nrows - 1, p.T, p.m, p.causal);
    const int64_t nwg = SAMPLE && !VARLEN ? (witness_count(p) + kSelGroup - 1) / kSelGroup : 0;
    const int64_t ngroups =
        SAMPLE ? (pmax > kFewCap ? kSampleGroups + nwg : 0) : (pmax + kSelGroup - 1) / kSelGroup;
    const int64_t nslab = (p.nrows + SQ - 1) / SQ;
    if (ngroups <= 0 || nslab <= 0) return hipSuccess;
    // about kTargetWaves waves in all, at most one per group of a slab
    const int64_t target = VARLEN ? kTargetWavesDocs : kTargetWaves;
    int64_t waves = (target + nslab - 1) / nslab;
    waves = waves < ngroups ? waves : ngroups;
    const int64_t blocks = ((waves + kRowsWaves - 1) / kRowsWaves + 7) / 8 * 8;
    hipLaunchKernelGGL((score_rows_kernel<DT, NB, D, SQ, VARLEN, SAMPLE>),
                       dim3((unsigned)blocks, (unsigned)nslab), dim3(kRowsThreads), 0, stream, p);
    return hipGetLastError();
}

template <int DT, int NB, int D>
hipError_t launch_sq(const ScoreSelectParams &p, bool varlen, bool sample, hipStream_t stream)
{
    if (sample)
        return varlen ? launch_rows<DT, NB, D, 1, true, true>(p, stream)
                      : launch_rows<DT, NB, D, 1, false, true>(p, stream);
    if (varlen) return launch_rows<DT, NB, D, 1, true, false>(p, stream);
    return p.nrows == 1 ? launch_rows<DT, NB, D, 1, false, false>(p, stream)
                        : launch_rows<DT, NB, D, 2, false, false>(p, stream);
}

}  // namespace

hipError_t launch_score_rows(int dtype, int nb, int d, bool varlen, bool sample,
                             const ScoreSelectParams &p, hipStream_t stream, bool *supported)
{
    *supported = true;
#define DSAI_CASE(DT, NB, D) \
    if (dtype == DT && nb == NB && d == D) return launch_sq<DT, NB, D>(p, varlen, sample, stream);
    DSAI_CASE(1, 1, 32) DSAI_CASE(1, 1, 64) DSAI_CASE(1, 1, 128)
    DSAI_CASE(1, 2, 32) DSAI_CASE(1, 2, 64) DSAI_CASE(1, 2, 128)
    DSAI_CASE(2, 1, 32) DSAI_CASE(2, 1, 64) DSAI_CASE(2, 1, 128)
    DSAI_CASE(2, 2, 32) DSAI_CASE(2, 2, 64) DSAI_CASE(2, 2, 128)
    DSAI_CASE(3, 1, 64) DSAI_CASE(3, 1, 128) DSAI_CASE(3, 2, 64) DSAI_CASE(3, 2, 128)
    DSAI_CASE(0, 1, 32) DSAI_CASE(0, 1, 64)
    DSAI_CASE(0, 2, 32) DSAI_CASE(0, 2, 64)
#undef DSAI_CASE
    *supported = false;
    return hipSuccess;
}

}  // namespace dsai
