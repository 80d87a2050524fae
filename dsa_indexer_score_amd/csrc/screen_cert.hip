// screen_cert: per-query DoSA score certificates and key norms for the
// screened streaming selection (gfx950).
//
// "DoSA: Dots Sparse Attention" (summary page, "Core method" and "Method
// steps"): a key whose score upper bound lies below a lower bound of the
// row's Ksel-th score cannot be selected.  For row t with head codes c_h,
// weights a_h = w_h * q_scale_h and a raw key vector k (k_scale multiplies
// the finished score), the exact score is sum_h a_h ReLU(c_h . k).  The
// certificate keeps 32 heads (one MFMA head block):
//  * head budget: if at most 32 heads are positive (a_h > 0), all of them
//    plus the negative heads of largest |a_h| ||c_h||; otherwise the 32
//    positive heads of largest a_h ||c_h||.  The page ranks negative heads by
//    |w_h| ||q_h|| min(p_h, 1 - p_h) with p_h a seed-set activation
//    frequency; no seed statistics are gathered here, so every p_h is taken
//    as 1/2, which leaves |w_h| ||q_h||;
//  * an omitted positive head h is bounded through the kept positive head j
//    maximising [c_h . c_j]_+ / ||c_j||: beta_h = [c_h . c_j]_+ / ||c_j||^2,
//    ReLU(c_h . k) <= beta_h ReLU(c_j . k) + ||c_h - beta_h c_j|| ||k||
//    (positive homogeneity, subadditivity, Cauchy-Schwarz), so a_h beta_h
//    folds into j's weight and a_h ||c_h - beta_h c_j|| into the allowance E;
//  * omitted negative heads are dropped (they only lower the score).
// Then U(k) = sum_kept wt_j ReLU(c_j . k) + E ||k|| >= score(k).  The page
// asks for bounds that hold in floating point (its conservative numerics);
// here the key-norm coefficient carries, besides E, a margin of
// 8 (d + 64) 2^-24 (sum_h |a_h| ||c_h|| + sum_kept (|wt_j| + fold_j) ||c_j||
// + E), well above the fp32 rounding of the score, of the bound and of the
// norms, all of which are at most a few (d + H) unit roundoffs of those
// magnitudes times ||k|| (each |c_h . k| <= ||c_h|| ||k||).
//
// One wave per row: the 64 x 64 head Gram matrix comes from 8 MFMAs per
// head-block pair on the same operands the scoring kernel uses; lane h then
// owns head h for the ranking, anchor search and residual norm.
#include "kernels.h"
#include "mfma_ops.h"

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
    __shared__ float fold[kHeadsMax], nrm[kHeadsMax];
    __shared__ int kept_pos[kHeadsMax];

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
    const float prio = fabsf(a) * n;
    const int np = __popcll(__ballot(pos));
    int rank = 0;  // among heads of the same sign class: larger priority, then lower index
    for (int j = 0; j < kHeadsMax; ++j) {
        const float pj = __shfl(prio, j);
        const bool posj = __shfl((int)pos, j) != 0;
        const bool vj = j < p.H;
        rank += (vj && posj == pos && (pj > prio || (pj == prio && j < h))) ? 1 : 0;
    }
    const bool kept = valid && (np <= kKept ? (pos || rank < kKept - np) : (pos && rank < kKept));

    // order: kept heads (by index), omitted heads, missing heads
    const uint64_t km = __ballot(kept), om = __ballot(valid && !kept), mm = __ballot(!valid);
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));  // lanes < h
    const int slot = kept ? __popcll(km & below)
                          : (valid ? __popcll(km) + __popcll(om & below)
                                   : __popcll(km) + __popcll(om) + __popcll(mm & below));
    p.cert_perm[r * kHeadsMax + slot] = valid ? h : -1;
    p.cert_w[r * kHeadsMax + slot] = a;

    // anchors of omitted positive heads and their folds
    nrm[h] = n;
    kept_pos[h] = kept && pos && nn > 0.f;
    fold[h] = 0.f;
    __syncthreads();
    const bool omit_pos = pos && !kept;
    float resid = 0.f;
    if (omit_pos) {
        int anc = -1;
        float best = -1.f;
        for (int j = 0; j < kHeadsMax; ++j) {
            if (!kept_pos[j]) continue;
            const float s = fmaxf(G[h][j], 0.f) / nrm[j];
            if (s > best) {
                best = s;
                anc = j;
            }
        }
        const float beta = anc >= 0 ? fmaxf(G[h][anc], 0.f) / G[anc][anc] : 0.f;
        float r2 = 0.f;
        for (int dd = 0; dd < D; ++dd) {
            const float x = cv[h][dd] - (anc >= 0 ? beta * cv[anc][dd] : 0.f);
            r2 = fmaf(x, x, r2);
        }
        resid = sqrtf(r2);
        if (anc >= 0) atomicAdd(&fold[anc], a * beta);
    }
    __syncthreads();
    const float E = wave_sum(omit_pos ? a * resid : 0.f);
    const float wt = kept ? a + fold[h] : 0.f;
    const float C = wave_sum(valid ? prio : 0.f);
    const float Ct = wave_sum(kept ? (fabsf(wt) + fold[h]) * n : 0.f) + E;
    const float mu = 8.f * (float)(D + kHeadsMax) * 0x1p-24f * (C + Ct);
    if (kept) p.cert_wt[r * kKept + slot] = wt;
    if (lane == 0) p.cert_e[r] = (E + mu) * (1.f + 0x1p-20f);
}

// ||k_j|| of the raw key codes (fp32), one thread per key.
template <int DT, int D>
__global__ void __launch_bounds__(256) key_norms_kernel(ScoreSelectParams p)
{
    using O = Op<DT, D>;
    using A = typename O::A;
    constexpr int KS = O::KS, ES = O::ES;
    constexpr int EPA = sizeof(A) / sizeof(float) == 4 ? 8 : 1;
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
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
