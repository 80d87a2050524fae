// screen_cert: per-query DoSA score certificates and key norms for the
// screened streaming selection (gfx950).
//
// "DoSA: Dots Sparse Attention" (summary page, "Core method", "Method steps"
// and "Technical novelty"): a key whose score upper bound lies below a lower
// bound of the row's Ksel-th score cannot be selected.  For row t with head
// codes c_h, weights a_h = w_h * q_scale_h and a raw key vector k (k_scale
// multiplies the finished score), the exact score is sum_h a_h ReLU(c_h . k).
// The certificate fills one MFMA head block of 32 rows:
//  * seed statistics: each head's activation frequency p_h, the share of a
//    seed set of the row's visible keys (256 keys spread evenly over them,
//    or all of them) with c_h . k > 0;
//  * head budget r (31 when the aggregate below takes a row, else 32): if
//    at most r heads are positive (a_h > 0), all of them plus the negative
//    heads of largest |a_h| ||c_h|| min(p_h, 1 - p_h); otherwise the r
//    positive heads of largest a_h ||c_h||;
//  * an omitted positive head h is bounded through the kept positive head j
//    maximising [c_h . c_j]_+ / ||c_j||: beta_h = [c_h . c_j]_+ / ||c_j||^2,
//    ReLU(c_h . k) <= beta_h ReLU(c_j . k) + ReLU(d_h . k) with the residual
//    d_h = c_h - beta_h c_j (positive homogeneity, subadditivity), so
//    a_h beta_h folds into j's weight; the residuals' sum
//    sum_h ReLU(a_h d_h . k) is at most E ||k|| with the joint allowance
//    E = (||sum u_h|| + sqrt(sum_{h,l} |u_h . u_l|)) / 2, u_h = a_h d_h
//    (also at most the per-head sum_h a_h ||d_h||, which is used when
//    smaller after rounding);
//  * omitted negative heads lower the score.  Those with p_h >= 1/2 (the
//    majority-active set A) lower it by at least ReLU(a_A . k) with
//    a_A = sum_{h in A} |a_h| c_h (subadditivity); a_A, rounded to the
//    operand type the MFMA reads (a~), takes the block's last row, with
//    bound weight -1 and exact weight 0, and ||a~ - a_A|| joins the
//    allowance.  It needs a free row: with H = 64 the 33 omitted heads
//    would not fit the second block, so there the budget stays 32 and
//    omitted negative heads are simply dropped.
// Then U(k) = sum_kept wt_j ReLU(c_j . k) - ReLU(a~ . k) + E' ||k|| >=
// score(k).  The page asks for bounds that hold in floating point (its
// conservative numerics); here the key-norm coefficient E' carries, besides
// E and ||a~ - a_A||, a margin of 8 (d + 64) 2^-24 (sum_h |a_h| ||c_h|| +
// sum_kept (|wt_j| + fold_j) ||c_j|| + E + ||a~||), well above the fp32
// rounding of the score, of the bound and of the norms, all of which are at
// most a few (d + H) unit roundoffs of those magnitudes times ||k|| (each
// |c . k| <= ||c|| ||k||).
//
// One wave per row: the 64 x 64 head Gram matrix comes from 8 MFMAs per
// head-block pair, the seed dots from 2 head blocks x 8 seed column blocks,
// on the same operands the scoring kernel uses; lane h then owns head h for
// the ranking, anchor search and residuals.
#include "kernels.h"
#include "mfma_ops.h"
#include "select_common.h"

namespace dsai {
namespace {

constexpr int kHeadsMax = 64;  // two head blocks
constexpr int kKept = 32;      // one head block

__device__ inline void operand_values(bf16x8 a, float *o)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (float)a[e];
}
__device__ inline void operand_values(float a, float *o) { o[0] = a; }

__device__ inline float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

template <int DT, int D>
__global__ void __launch_bounds__(64) certificate_kernel(ScoreSelectParams p)
{
    using O = Op<DT, D>;
    using A = typename O::A;
    constexpr int KS = O::KS, ES = O::ES;
    constexpr int EPA = sizeof(A) / sizeof(float) == 4 ? 8 : 1;  // values per operand
    __shared__ float G[kHeadsMax][kHeadsMax + 1];
    __shared__ float cv[kHeadsMax][D + 1];
    __shared__ float fold[kHeadsMax], nrm[kHeadsMax], wsh[kHeadsMax];
    __shared__ int kept_pos[kHeadsMax], act[kHeadsMax];

    const int lane = threadIdx.x, hh = lane >> 5, l32 = lane & 31;
    const int64_t r = blockIdx.x;  // row within the launch
    const int64_t t = p.row0 + r;
    const char *qbytes = static_cast<const char *>(p.q);

    // head codes as MFMA operands (missing heads are zero rows) and as floats
    A qa[2][KS];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int head = 32 * b + l32;
        const bool ok = head < p.H;
        O::load_a(qbytes + ((t * p.H + (ok ? head : 0)) * (int64_t)D) * ES, hh, qa[b]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (!ok) qa[b][ks] = O::zero();
            float v[EPA];
            operand_values(qa[b][ks], v);
#pragma unroll
            for (int e = 0; e < EPA; ++e) cv[head][hh * (D / 2) + ks * EPA + e] = v[e];
        }
    }
    // Gram matrix G[i][j] = c_i . c_j
#pragma unroll
    for (int b1 = 0; b1 < 2; ++b1)
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
            f32x16 acc;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = O::mma(qa[b1][ks], qa[b2][ks], acc);
#pragma unroll
            for (int v = 0; v < 16; ++v)
                G[32 * b1 + 8 * (v >> 2) + 4 * hh + (v & 3)][32 * b2 + l32] = acc[v];
        }
    __syncthreads();

    // ---- seed statistics: each head's activation frequency p_h on a seed
    // set of the row's visible keys (n_s = min(P, 256) keys at j = i P / n_s)
    constexpr int kSeeds = 256;
    int64_t P = 0;
    if (p.k && p.T > 0) P = visible_keys(p.q_pos0 + t, p.T, p.m, p.causal);
    const int ns = P < kSeeds ? (int)P : kSeeds;
    act[lane] = 0;
    __syncthreads();
    if (ns > 0) {
        const char *kbytes = static_cast<const char *>(p.k);
        constexpr int64_t ROWB = (int64_t)D * ES;
        for (int cb = 0; cb < kSeeds / 32 && cb * 32 < ns; ++cb) {
            const int i = cb * 32 + l32;
            const bool ok = i < ns;
            const int64_t j = ok ? (int64_t)i * P / ns : 0;
            A bk[KS];
            O::load_a(kbytes + j * ROWB, hh, bk);  // a key row as B (same slot map)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                f32x16 acc;
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) acc = O::mma(qa[b][ks], bk[ks], acc);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    // row (head) 32 b + 8 (v/4) + 4 hh + v%4, column (seed) l32
                    const uint64_t m = __ballot(ok && acc[v] > 0.f);
                    if (lane == 0) {
                        act[32 * b + 8 * (v >> 2) + (v & 3)] += __popcll(m & 0xFFFFFFFFull);
                        act[32 * b + 8 * (v >> 2) + 4 + (v & 3)] += __popcll(m >> 32);
                    }
                }
            }
        }
    }
    __syncthreads();

    // lane h owns head h
    const int h = lane;
    const bool valid = h < p.H;
    float a = 0.f;
    if (valid) {
        a = p.w[t * p.w_stride + h];
        if (DT == 2) a *= p.q_scale[t * p.H + h];
    }
    const float nn = G[h][h];
    const float n = sqrtf(nn);
    const bool pos = valid && a > 0.f;
    // negative heads rank by |a_h| ||c_h|| min(p_h, 1 - p_h); with no seeds
    // every p_h is taken as 1/2
    const int ah = act[h];
    const float ph = ns > 0 ? (float)ah / (float)ns : 0.5f;
    const float prio = pos ? fabsf(a) * n : fabsf(a) * n * fminf(ph, 1.f - ph);
    // the aggregate of the omitted majority-active negative heads takes one
    // row of the kept block when the omitted heads then still fit one block
    const bool agg_on = p.H <= 2 * kKept - 1 && ns > 0;
    const int r_budget = agg_on ? kKept - 1 : kKept;
    const int np = __popcll(__ballot(pos));
    int rank = 0;  // among heads of the same sign class: larger priority, then lower index
    for (int j = 0; j < kHeadsMax; ++j) {
        const float pj = __shfl(prio, j);
        const bool posj = __shfl((int)pos, j) != 0;
        const bool vj = j < p.H;
        rank += (vj && posj == pos && (pj > prio || (pj == prio && j < h))) ? 1 : 0;
    }
    const bool kept =
        valid && (np <= r_budget ? (pos || rank < r_budget - np) : (pos && rank < r_budget));
    // majority-active omitted negative heads (2 act >= n_s: p_h >= 1/2)
    const bool in_agg = agg_on && valid && !kept && a < 0.f && 2 * ah >= ns;

    // order: kept heads (by index), [the aggregate], omitted heads, missing heads
    const uint64_t km = __ballot(kept), om = __ballot(valid && !kept), mm = __ballot(!valid);
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));  // lanes < h
    const int nk = agg_on ? kKept : __popcll(km);  // slots before the omitted heads
    const int slot = kept ? __popcll(km & below)
                          : (valid ? nk + __popcll(om & below)
                                   : nk + __popcll(om) + __popcll(mm & below));
    // with the aggregate there is one slot fewer than lanes: the last
    // missing head (there is one, as H <= 63) has none
    if (slot < kHeadsMax) {
        p.cert_perm[r * kHeadsMax + slot] = valid ? h : -1;
        p.cert_w[r * kHeadsMax + slot] = a;
    }
    if (agg_on && lane == 0) {
        p.cert_perm[r * kHeadsMax + kKept - 1] = kAggSlot;
        p.cert_w[r * kHeadsMax + kKept - 1] = 0.f;  // not part of the exact score
    }
    if (p.cert_act) p.cert_act[r * kHeadsMax + h] = valid ? ah : 0;

    // anchors of omitted positive heads and their folds
    nrm[h] = n;
    wsh[h] = a;
    kept_pos[h] = kept && pos && nn > 0.f;
    fold[h] = 0.f;
    __syncthreads();
    const bool omit_pos = pos && !kept;
    float resid = 0.f;
    int anc = -1;
    float beta = 0.f;
    if (omit_pos) {
        float best = -1.f;
        for (int j = 0; j < kHeadsMax; ++j) {
            if (!kept_pos[j]) continue;
            const float sj = fmaxf(G[h][j], 0.f) / nrm[j];
            if (sj > best) {
                best = sj;
                anc = j;
            }
        }
        beta = anc >= 0 ? fmaxf(G[h][anc], 0.f) / G[anc][anc] : 0.f;
        float r2 = 0.f;
        for (int dd = 0; dd < D; ++dd) {
            const float x = cv[h][dd] - (anc >= 0 ? beta * cv[anc][dd] : 0.f);
            r2 = fmaf(x, x, r2);
        }
        resid = sqrtf(r2);
        if (anc >= 0) atomicAdd(&fold[anc], a * beta);
    }
    __syncthreads();
    // the residuals d_h = c_h - beta_h c_anchor overwrite the omitted positive
    // heads' rows (no anchor and no aggregate head is one of them)
    if (omit_pos)
        for (int dd = 0; dd < D; ++dd) cv[h][dd] -= anc >= 0 ? beta * cv[anc][dd] : 0.f;
    __syncthreads();
    const float E = wave_sum(omit_pos ? a * resid : 0.f);
    // joint residual bound (DoSA summary, "Technical novelty"): with
    // u_h = a_h d_h, sum_h [u_h . k]_+ <= (||sum u_h|| + sqrt(sum |u_h . u_l|)) / 2 ||k||
    const uint64_t opm = __ballot(omit_pos);
    float pair = 0.f;
    if (omit_pos) {
        for (uint64_t mrest = opm; mrest; mrest &= mrest - 1) {
            const int l = __ffsll((unsigned long long)mrest) - 1;
            float dot = 0.f;
            for (int dd = 0; dd < D; ++dd) dot = fmaf(cv[h][dd], cv[l][dd], dot);
            pair += fabsf(a * wsh[l] * dot);
        }
    }
    const float S2 = wave_sum(pair);
    float vs2 = 0.f;
    for (int dd = lane; dd < D; dd += 64) {
        float sdd = 0.f;
        for (uint64_t mrest = opm; mrest; mrest &= mrest - 1) {
            const int l = __ffsll((unsigned long long)mrest) - 1;
            sdd = fmaf(wsh[l], cv[l][dd], sdd);
        }
        vs2 = fmaf(sdd, sdd, vs2);
    }
    const float Ej = 0.5f * (sqrtf(wave_sum(vs2)) + sqrtf(S2));
    const float Euse = fminf(E, Ej);

    // the aggregate a_A = sum_{h in A} |a_h| c_h, rounded to the operand type
    // the MFMA reads (bf16; fp32 unchanged); ||a~ - a_A|| widens the
    // allowance, ||a~|| the rounding margin
    const uint64_t agm = __ballot(in_agg);
    float d2 = 0.f, g2 = 0.f;
    if (agg_on) {
        for (int dd = lane; dd < D; dd += 64) {
            float x = 0.f;
            for (uint64_t mrest = agm; mrest; mrest &= mrest - 1) {
                const int l = __ffsll((unsigned long long)mrest) - 1;
                x = fmaf(fabsf(wsh[l]), cv[l][dd], x);
            }
            const float xr = DT == 0 ? x : (float)(__bf16)x;
            p.cert_agg[r * D + dd] = xr;
            d2 = fmaf(xr - x, xr - x, d2);
            g2 = fmaf(xr, xr, g2);
        }
    }
    const float delta = sqrtf(wave_sum(d2)), gnorm = sqrtf(wave_sum(g2));

    const float wt = kept ? a + fold[h] : 0.f;
    const float C = wave_sum(valid ? fabsf(a) * n : 0.f);
    const float Ct = wave_sum(kept ? (fabsf(wt) + fold[h]) * n : 0.f) + E + gnorm;
    const float mu = 8.f * (float)(D + kHeadsMax) * 0x1p-24f * (C + Ct);
    if (kept) p.cert_wt[r * kKept + slot] = wt;
    if (agg_on && lane == 0) p.cert_wt[r * kKept + kKept - 1] = -1.f;  // subtracts [a~ . k]_+
    if (lane == 0) p.cert_e[r] = (Euse + delta + mu) * (1.f + 0x1p-20f);
}

// ||k_j|| of the raw key codes (fp32), one thread per key; the first
// launch of a screened call, so it also zeroes the call's statistics.
template <int DT, int D>
__global__ void __launch_bounds__(256) key_norms_kernel(ScoreSelectParams p)
{
    using O = Op<DT, D>;
    using A = typename O::A;
    constexpr int KS = O::KS, ES = O::ES;
    constexpr int EPA = sizeof(A) / sizeof(float) == 4 ? 8 : 1;
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p.scr_stats && j < 2) p.scr_stats[j] = 0;  // the call's screening statistics
    if (j >= p.T) return;
    const char *row = static_cast<const char *>(p.k) + j * (int64_t)D * ES;
    float s = 0.f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        A b[KS];
        O::load_a(row, half, b);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float v[EPA];
            operand_values(b[ks], v);
#pragma unroll
            for (int e = 0; e < EPA; ++e) s = fmaf(v[e], v[e], s);
        }
    }
    p.knorm[j] = sqrtf(s);
}

}  // namespace

hipError_t launch_certificates(int dtype, int d, const ScoreSelectParams &p, hipStream_t stream,
                               bool *supported)
{
    *supported = p.H > 32 && p.H <= kHeadsMax;
    if (!*supported || p.nrows <= 0) return hipSuccess;
#define DSAI_CASE(DT, D)                                                                     \
    if (dtype == DT && d == D) {                                                             \
        hipLaunchKernelGGL((certificate_kernel<DT, D>), dim3((unsigned)p.nrows), dim3(64), 0, \
                           stream, p);                                                       \
        return hipGetLastError();                                                            \
    }
    DSAI_CASE(1, 32) DSAI_CASE(1, 64) DSAI_CASE(1, 128)
    DSAI_CASE(2, 32) DSAI_CASE(2, 64) DSAI_CASE(2, 128)
    DSAI_CASE(0, 32) DSAI_CASE(0, 64)
#undef DSAI_CASE
    *supported = false;
    return hipSuccess;
}

hipError_t launch_key_norms(int dtype, int d, const ScoreSelectParams &p, hipStream_t stream,
                            bool *supported)
{
    *supported = true;
    if (p.T <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)((p.T + 255) / 256);
#define DSAI_CASE(DT, D)                                                                       \
    if (dtype == DT && d == D) {                                                               \
        hipLaunchKernelGGL((key_norms_kernel<DT, D>), dim3(blocks), dim3(256), 0, stream, p); \
        return hipGetLastError();                                                              \
    }
    DSAI_CASE(1, 32) DSAI_CASE(1, 64) DSAI_CASE(1, 128)
    DSAI_CASE(2, 32) DSAI_CASE(2, 64) DSAI_CASE(2, 128)
    DSAI_CASE(0, 32) DSAI_CASE(0, 64)
#undef DSAI_CASE
    *supported = false;
    return hipSuccess;
}

}  // namespace dsai
