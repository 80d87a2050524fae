/*
 * CPU ORACLE for the lightning-indexer step.  TEST INFRASTRUCTURE ONLY:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  It shares no code with the HIP library and must never be
 * reached from the product path.
 *
 * What it computes (plain definition, fp64, no blocking or reordering):
 *
 *   score  s_tj = sum_h w_h * ReLU(q_{t,h} . k_j)
 *          -- DoSA: Dots Sparse Attention (summary page), "Prerequisites:
 *             DSA and the multi-head indexer": signed head weights w_h,
 *             [.]_+ is ReLU, all visible keys are scored.
 *   select the top-k visible keys; total order: higher score first, equal
 *          scores to the lower key index (the "unified tie rule" that page
 *          leaves unstated, taken as higher score then lower index).
 *   visibility -- GLM-5.3-Flash Module 06 "DSA & KPool", section 3
 *          (Causality): position p sees token j iff j <= p; a pool of m
 *          tokens becomes selectable only once its last token is visible,
 *          so pool j is visible iff (j+1)*m - 1 <= p.
 *   expansion and tail -- same module, section 2 (selection budget): each
 *          selected pool expands to its m positions; the still-incomplete
 *          pool (at most m-1 positions, p+1 mod m of them) is appended as
 *          a visible tail; buffers are topk + m - 1 wide, padded.
 *   canonical order -- Adjacent-Query KV-Index Overlap in 256K DSA
 *          Training, section 3: consumers see the indices sorted by KV index.
 *
 * Inputs are dequantised exactly: fp32 as is, bf16 and OCP e4m3 (e4m3fn)
 * decoded by hand from their bit fields, times the per-row fp32 scale when
 * one is given.  Every score is a naive h-outer, i-inner double loop; the
 * selection is a full qsort of (score, index) pairs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_E4M3 = 2 };

/* bf16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double oracle_decode_bf16(uint16_t b)
{
    int sign = (b >> 15) & 1, e = (b >> 7) & 0xFF, f = b & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)f, -126 - 7);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(128.0 + (double)f, e - 127 - 7);
    return sign ? -v : v;
}

/* OCP e4m3 (e4m3fn): 1 sign, 4 exponent (bias 7), 3 fraction bits; no
 * infinities; S.1111.111 is NaN; largest finite magnitude 448. */
double oracle_decode_e4m3(uint8_t b)
{
    int sign = (b >> 7) & 1, e = (b >> 3) & 0xF, f = b & 7;
    double v;
    if (e == 15 && f == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)f, -6 - 3);
    else
        v = ldexp(8.0 + (double)f, e - 7 - 3);
    return sign ? -v : v;
}

double oracle_decode_f32(uint32_t b)
{
    float f;
    memcpy(&f, &b, 4);
    return (double)f;
}

static double elem(const void *base, int dtype, int64_t i)
{
    switch (dtype) {
    case OR_F32: return oracle_decode_f32(((const uint32_t *)base)[i]);
    case OR_BF16: return oracle_decode_bf16(((const uint16_t *)base)[i]);
    case OR_E4M3: return oracle_decode_e4m3(((const uint8_t *)base)[i]);
    }
    return NAN;
}

/* Output width: topk slots, plus m-1 tail slots when the tail is on. */
int oracle_output_width(int topk, int m, int expand, int tail)
{
    return topk + ((expand && tail) ? (m - 1) : 0);
}

/* Visible keys and tail length for absolute position p. */
static void visibility(int64_t p, int64_t T, int m, int causal, int expand, int tail,
                       int64_t *P, int64_t *r)
{
    if (!causal) {
        *P = T;
        *r = 0;
        return;
    }
    int64_t complete = (p + 1) / m; /* pools whose last token is <= p */
    *P = complete < T ? complete : T;
    *r = (expand && tail) ? (p + 1) - (*P) * m : 0;
}

typedef struct {
    double s;
    int64_t j;
} scored_key;

static int by_rank(const void *a, const void *b)
{
    const scored_key *x = (const scored_key *)a, *y = (const scored_key *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int by_value(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Dequantised key matrix [T, d] in fp64. */
static double *dequant_keys(const void *k, const float *k_scale, int dtype, int64_t T, int d)
{
    double *K = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * (size_t)d);
    if (!K) return NULL;
    for (int64_t j = 0; j < T; ++j) {
        double sc = k_scale ? (double)k_scale[j] : 1.0;
        for (int i = 0; i < d; ++i)
            K[j * d + i] = elem(k, dtype, j * d + i) * sc;
    }
    return K;
}

static void dequant_query(const void *q, const float *q_scale, const float *w, int64_t w_stride,
                          int dtype, int64_t r, int H, int d, double *Q, double *Wt)
{
    for (int h = 0; h < H; ++h) {
        double sc = q_scale ? (double)q_scale[r * H + h] : 1.0;
        for (int i = 0; i < d; ++i)
            Q[h * d + i] = elem(q, dtype, (r * H + h) * (int64_t)d + i) * sc;
        Wt[h] = (double)w[r * w_stride + h];
    }
}

/* The score of one (query, key) pair: sum over heads of w_h * max(0, q_h . k). */
static double score_one(const double *Q, const double *Wt, const double *Kj, int H, int d)
{
    double s = 0.0;
    for (int h = 0; h < H; ++h) {
        double dot = 0.0;
        for (int i = 0; i < d; ++i)
            dot += Q[h * d + i] * Kj[i];
        s += Wt[h] * (dot > 0.0 ? dot : 0.0);
    }
    return s;
}

/*
 * Select rows.  Row r of the gathered inputs (q + r*H*d, q_scale + r*H,
 * w + r*w_stride) sits at absolute sequence position pos[r].
 * Outputs per row r:
 *   idx[r*W ..]        final row: expanded, tail appended, sorted ascending, -1 padded
 *   valid_len[r]
 *   key_idx[r*Ksel ..] selected keys in rank order (best first), -1 padded
 *   key_score[r*Ksel ..] their fp64 scores
 *   n_sel[r]           number of selected keys
 *   tau[r]             score of the last selected key (NaN when none)
 * Returns 0, or -1 (bad arguments / allocation), -2 (tail longer than m-1:
 * T does not cover every complete pool), -3 (non-finite score).
 */
int oracle_select_rows(const void *q, const float *q_scale, const float *w, int64_t w_stride,
                       const void *k, const float *k_scale, int dtype, int64_t nrows,
                       const int64_t *pos, int64_t T, int H, int d, int m, int topk,
                       int causal, int expand, int tail, int32_t *idx, int32_t *valid_len,
                       int32_t *key_idx, double *key_score, int32_t *n_sel, double *tau,
                       int nthreads)
{
    if (nrows < 0 || T < 0 || H < 1 || d < 1 || m < 1 || topk < 1) return -1;
    if (expand && topk % m) return -1;
    const int W = oracle_output_width(topk, m, expand, tail);
    const int Ksel = expand ? topk / m : topk;
    double *K = dequant_keys(k, k_scale, dtype, T, d);
    if (!K) return -1;
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double *Q = (double *)malloc(sizeof(double) * (size_t)H * d);
        double *Wt = (double *)malloc(sizeof(double) * (size_t)H);
        scored_key *cand = (scored_key *)malloc(sizeof(scored_key) * (size_t)(T > 0 ? T : 1));
        int32_t *row = (int32_t *)malloc(sizeof(int32_t) * (size_t)(W > 0 ? W : 1));
        if (!Q || !Wt || !cand || !row) status = -1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t r = 0; r < nrows; ++r) {
            if (status) continue;
            int64_t P, tl;
            visibility(pos[r], T, m, causal, expand, tail, &P, &tl);
            if (tl > m - 1 || tl < 0) { status = -2; continue; }
            dequant_query(q, q_scale, w, w_stride, dtype, r, H, d, Q, Wt);
            for (int64_t j = 0; j < P; ++j) {
                cand[j].s = score_one(Q, Wt, K + j * d, H, d);
                cand[j].j = j;
                if (!isfinite(cand[j].s)) status = -3;
            }
            qsort(cand, (size_t)P, sizeof(scored_key), by_rank);
            int64_t n = P < Ksel ? P : Ksel;
            n_sel[r] = (int32_t)n;
            tau[r] = n > 0 ? cand[n - 1].s : NAN;
            for (int64_t i = 0; i < Ksel; ++i) {
                key_idx[r * Ksel + i] = i < n ? (int32_t)cand[i].j : -1;
                key_score[r * Ksel + i] = i < n ? cand[i].s : NAN;
            }
            int64_t cnt = 0;
            const int mexp = expand ? m : 1;
            for (int64_t i = 0; i < n; ++i)
                for (int e = 0; e < mexp; ++e)
                    row[cnt++] = (int32_t)(cand[i].j * mexp + e);
            for (int64_t e = 0; e < tl; ++e)
                row[cnt++] = (int32_t)(P * m + e);
            qsort(row, (size_t)cnt, sizeof(int32_t), by_value);
            for (int64_t i = 0; i < W; ++i)
                idx[r * W + i] = i < cnt ? row[i] : -1;
            valid_len[r] = (int32_t)cnt;
        }
        free(Q);
        free(Wt);
        free(cand);
        free(row);
    }
    free(K);
    return status;
}

/* fp64 scores of arbitrary (row, key) pairs; row r as in oracle_select_rows. */
int oracle_pair_scores(const void *q, const float *q_scale, const float *w, int64_t w_stride,
                       const void *k, const float *k_scale, int dtype, int64_t T, int H, int d,
                       int64_t n, const int64_t *row, const int64_t *key, double *out,
                       int nthreads)
{
    if (n < 0 || H < 1 || d < 1) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double *Q = (double *)malloc(sizeof(double) * (size_t)H * d);
        double *Wt = (double *)malloc(sizeof(double) * (size_t)H);
        double *Kj = (double *)malloc(sizeof(double) * (size_t)d);
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t e = 0; e < n; ++e) {
            int64_t j = key[e];
            if (!Q || !Wt || !Kj || j < 0 || j >= T) { out[e] = NAN; continue; }
            dequant_query(q, q_scale, w, w_stride, dtype, row[e], H, d, Q, Wt);
            double sc = k_scale ? (double)k_scale[j] : 1.0;
            for (int i = 0; i < d; ++i)
                Kj[i] = elem(k, dtype, j * d + i) * sc;
            out[e] = score_one(Q, Wt, Kj, H, d);
        }
        free(Q);
        free(Wt);
        free(Kj);
    }
    return 0;
}

/* Condition sums B(row, key) = sum_h |w_h| * sum_i |q_hi * k_i| of arbitrary
 * pairs: the standard error bound of evaluating a score in floating point
 * with unit roundoff u over n sequential operations is gamma_n * B, with
 * gamma_n = n u / (1 - n u).  Used to derive the fp32 tolerance. */
int oracle_pair_bounds(const void *q, const float *q_scale, const float *w, int64_t w_stride,
                       const void *k, const float *k_scale, int dtype, int64_t T, int H, int d,
                       int64_t n, const int64_t *row, const int64_t *key, double *out,
                       int nthreads)
{
    if (n < 0 || H < 1 || d < 1) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double *Q = (double *)malloc(sizeof(double) * (size_t)H * d);
        double *Wt = (double *)malloc(sizeof(double) * (size_t)H);
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t e = 0; e < n; ++e) {
            int64_t j = key[e];
            if (!Q || !Wt || j < 0 || j >= T) { out[e] = NAN; continue; }
            dequant_query(q, q_scale, w, w_stride, dtype, row[e], H, d, Q, Wt);
            double sc = k_scale ? (double)k_scale[j] : 1.0, b = 0.0;
            for (int h = 0; h < H; ++h) {
                double a = 0.0;
                for (int i = 0; i < d; ++i)
                    a += fabs(Q[h * d + i] * elem(k, dtype, j * d + i) * sc);
                b += fabs(Wt[h]) * a;
            }
            out[e] = b;
        }
        free(Q);
        free(Wt);
    }
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
