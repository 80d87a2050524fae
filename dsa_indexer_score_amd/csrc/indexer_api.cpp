// Host side of the C ABI declared in include/dsa_indexer.h: argument checks,
// output-width and workspace arithmetic, the query-chunk loop and launches.
// Nothing here computes scores or selections; every step of the indexer runs
// in the HIP kernels (score_select.hip, score_rows.hip, select_few.hip,
// pair_overlap.hip).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "dsa_indexer.h"
#include "kernels.h"

struct indexer_s {
    indexer_config cfg;
    int device;
};

namespace {

thread_local std::string g_hip_error;
thread_local std::string g_detail;  // why the last IDX_EWORKSPACE was returned, if known
thread_local std::string g_msg;

int fail_hip(hipError_t e)
{
    g_hip_error = hipGetErrorString(e);
    return IDX_EHIP;
}

constexpr int kAllFlags = IDX_EXPAND | IDX_TAIL | IDX_SCREEN | IDX_FP8_MFMA;
constexpr int64_t kMaxSel = 16000;  // 16-bit histogram counters bound the buffer at 65535

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

bool dtype_ok(int dt) { return dt == IDX_F32 || dt == IDX_BF16 || dt == IDX_FP8_E4M3; }

bool shape_supported(int dtype, int H, int d)
{
    if (H < 1 || H > 64) return false;
    switch (dtype) {
    case IDX_F32: return d == 32 || d == 64;
    case IDX_BF16: return d == 32 || d == 64 || d == 128;
    case IDX_FP8_E4M3: return d == 32 || d == 64 || d == 128;
    }
    return false;
}

int64_t ksel_of(int topk, int m, int flags) { return (flags & IDX_EXPAND) ? topk / m : topk; }

// Candidate slots per query.  With the running threshold a query appends
// about Ksel * (1 + ln(visible / Ksel)) candidates (plus histogram-bin slack),
// so 10 * Ksel slots hold every append for visible / Ksel up to several
// thousand and the compaction fallback stays rare; never more than every
// visible key plus one group, and at most 65472 (16-bit histogram counters).
int64_t capacity(int64_t ksel, int64_t pmax)
{
    const int64_t g = dsai::kSelGroup;
    int64_t cap = std::min<int64_t>(round_up(10 * ksel + 4 * g, g), 65472);
    int64_t all = round_up(std::max<int64_t>(pmax, 0), g) + g;
    return std::min(cap, all);
}

// Rows per streaming launch: query_chunk, or by default as many rows as
// 4 GiB of candidate buffers hold at the capacity T allows (so the size does
// not depend on the call's positions), and at least 2,048 (256 blocks).
// Results do not depend on the chunking.
constexpr int64_t kStreamAutoBytes = int64_t(1) << 32;
int64_t rows_per_launch(const indexer_config &cfg, int64_t S, int64_t cap_max)
{
    if (cfg.query_chunk > 0) return cfg.query_chunk < S ? cfg.query_chunk : S;
    int64_t r = kStreamAutoBytes / (cap_max * (int64_t)sizeof(uint2));
    r = std::max<int64_t>(r / dsai::kQueriesPerBlock * dsai::kQueriesPerBlock, 2048);
    return std::min(r, S);
}

// Rows at or below which the few-query path is taken by default: the
// streaming grid has one block per 8 rows, so below about 2,048 rows it
// leaves CUs idle; measured on decode-shaped rows at 65,536 and 262,144
// keys, the few-query path is faster up to 1,024 rows (1.4x-8.7x) and the
// streaming path from 1,536 on (by 8-25 %).
constexpr int64_t kFewRowsDefault = 1024;
// Packed documents with several rows each score each row's keys on its own
// on the few-query path, while the streaming path shares a staged key tile
// among a block's 8 rows: there the default stays at 64 rows unless there
// are at most two rows per document (batched decode).
constexpr int64_t kFewRowsDocsDefault = 64;
constexpr int64_t kFewMaxBytes = int64_t(1) << 32;
constexpr int64_t kFillBlocks = 256;  // one scoring block per CU (measured best)
constexpr int64_t kRowsKernelMax = 2;  // rows scored with q in registers, keys from HBM

// Few-query workspace for R rows of at most Tk keys each: the rows' key
// sample and witness scores [R, kSampStride] (f32), threshold estimates [R] (u32), candidate
// sub-list counts [R, kFewSub] (u32), repair marks [R] (i32), the directory
// of candidate batches [R, nbatch] of (offset, count), and the candidate
// sub-lists [R, cap] of (score bits, key), each 256-byte aligned.  cap also holds the
// streaming kernel's candidates when a row goes to the repair launch.  No
// part holds a score per key: the directory has one entry per kFewBatch
// keys, everything else is per row.
struct FewLayout {
    int64_t nbatch, cap, est, cnt, stat, dir, cand, bytes;
    FewLayout(int64_t R, int64_t Tk, int64_t ksel)
    {
        nbatch = (std::max<int64_t>(Tk, 1) + dsai::kFewBatch - 1) / dsai::kFewBatch;
        cap = std::max<int64_t>(dsai::kFewSub * dsai::kFewSubCap, capacity(ksel, Tk));
        est = round_up(R * dsai::kSampStride * 4, 256);
        cnt = est + round_up(R * 4, 256);
        stat = cnt + round_up(R * dsai::kFewSub * 4, 256);
        dir = stat + round_up(R * 4, 256);
        cand = dir + round_up(R * nbatch * 8, 256);
        bytes = cand + R * cap * 8;
    }
};

// Few-query path: at most the configured number of rows (ndoc < 0: a plain
// call, else the packed documents' count), and one row's layout fits.
bool use_few(const indexer_config &cfg, int64_t S, int64_t T, int64_t ksel, int64_t ndoc = -1)
{
    int64_t lim = cfg.few_query_rows;
    if (lim == 0) lim = ndoc < 0 || S <= 2 * ndoc ? kFewRowsDefault : kFewRowsDocsDefault;
    return lim > 0 && S <= lim && S <= 65535 && FewLayout(1, T, ksel).bytes <= kFewMaxBytes;
}

// Rows per few-query pass: all S while the workspace stays within 4 GiB,
// else as many as fit (the rows are then taken in several passes).
int64_t few_rows(int64_t S, int64_t T, int64_t ksel)
{
    int64_t lo = 1, hi = std::max<int64_t>(S, 1);  // largest r whose layout fits
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if (FewLayout(mid, T, ksel).bytes <= kFewMaxBytes) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Screening (IDX_SCREEN) on the streaming path: needs two head blocks.
bool use_screen(const indexer_config &cfg, int H)
{
    return (cfg.flags & IDX_SCREEN) && H > 32 && H <= 64;
}

// Streaming workspace: the candidate buffers [rows, cap] of (score bits,
// key); with screening, the call's statistics (two u64: keys tested against
// the bound, keys that passed) first, then the candidate buffers, the
// certificates of one launch's rows (head order [rows, 64] i32, weights
// [rows, 64], bound weights [rows, 32], key norm coefficient [rows],
// aggregate row [rows, 128]) and the key norms [T], each 256-byte aligned.
struct StreamLayout {
    int64_t cand = 0, perm, w, wt, e, agg, knorm, bytes;
    StreamLayout(int64_t rows, int64_t cap, int64_t T, bool screen)
    {
        bytes = rows * cap * (int64_t)sizeof(uint2);
        if (!screen) return;
        cand = 256;  // the call's screening statistics come first
        bytes += cand;
        perm = round_up(bytes, 256);
        w = perm + round_up(rows * 64 * 4, 256);
        wt = w + round_up(rows * 64 * 4, 256);
        e = wt + round_up(rows * 32 * 4, 256);
        agg = e + round_up(rows * 4, 256);
        knorm = agg + round_up(rows * 128 * 4, 256);
        bytes = knorm + std::max<int64_t>(T, 1) * 4;
    }
};

int64_t workspace_need(const indexer_config &cfg, int64_t S, int64_t T, int H, int64_t ksel,
                       int64_t pmax)
{
    if (use_few(cfg, S, T, ksel)) return FewLayout(few_rows(S, T, ksel), T, ksel).bytes;
    return StreamLayout(rows_per_launch(cfg, S, capacity(ksel, T)), capacity(ksel, pmax), T,
                        use_screen(cfg, H)).bytes;
}

struct DeviceGuard {
    int prev = -1;
    bool changed = false;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev)
    {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) {
            err = hipSetDevice(dev);
            changed = err == hipSuccess;
        }
    }
    ~DeviceGuard()
    {
        if (changed) (void)hipSetDevice(prev);
    }
};

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

int indexer_create(const indexer_config *cfg, int device, indexer_t *out)
{
    if (!cfg || !out || device < 0) return IDX_EINVAL;
    if (!dtype_ok(cfg->dtype)) return IDX_EINVAL;
    if (cfg->flags & ~kAllFlags) return IDX_EINVAL;
    if ((cfg->flags & IDX_TAIL) && !(cfg->flags & IDX_EXPAND)) return IDX_EINVAL;
    if (cfg->query_chunk < 0) return IDX_EINVAL;
    indexer_s *h = new (std::nothrow) indexer_s;
    if (!h) return IDX_EINVAL;
    h->cfg = *cfg;
    h->device = device;
    *out = h;
    return IDX_OK;
}

int indexer_destroy(indexer_t h)
{
    delete h;
    return IDX_OK;
}

int indexer_output_width(int topk, int m, int flags, int *W)
{
    if (!W || topk < 1 || m < 1 || (flags & ~kAllFlags))
        return IDX_EINVAL;
    if ((flags & IDX_TAIL) && !(flags & IDX_EXPAND)) return IDX_EINVAL;
    if ((flags & IDX_EXPAND) && topk % m) return IDX_EINVAL;
    int64_t w = (int64_t)topk + ((flags & IDX_TAIL) ? (m - 1) : 0);
    if (w > INT32_MAX) return IDX_EINVAL;
    *W = (int)w;
    return IDX_OK;
}

int indexer_workspace_bytes(indexer_t h, int64_t S, int64_t T, int H, int d, int m, int topk,
                            size_t *bytes)
{
    if (!h || !bytes || S < 0 || T < 0 || H < 1 || d < 1 || m < 1 || topk < 1) return IDX_EINVAL;
    if ((h->cfg.flags & IDX_EXPAND) && topk % m) return IDX_EINVAL;
    const int64_t ksel = ksel_of(topk, m, h->cfg.flags);
    if (ksel > kMaxSel) return IDX_EUNSUPPORTED;
    *bytes = (size_t)workspace_need(h->cfg, S, T, H, ksel, T);
    return IDX_OK;
}

}  // extern "C"

namespace {

struct Docs {  // packed-document layout (varlen); on = false: one document
    bool on = false;
    const int32_t *cu_q = nullptr, *cu_k = nullptr, *cu_tok = nullptr;
    const int64_t *pos0 = nullptr;
    int ndoc = 0;
    int64_t row_keys = 0;  // keys per row of the few-query path
};

struct Witness {  // earlier selections of the rows (few-query path only)
    const int32_t *ptr = nullptr;
    int64_t stride = 0;
    int n = 0;
};

// Keys per few-query row for packed documents: the caller's bound on a
// document's keys (0: unknown), at most T.
int64_t doc_row_keys(int64_t max_doc_keys, int64_t T)
{
    return max_doc_keys > 0 && max_doc_keys < T ? max_doc_keys : T;
}

// Largest rows r (a multiple of the block's 8 queries unless r = S < 8) whose
// layout bytes(r) fit in `avail`; 0 when not even the smallest fits.
template <class F> int64_t rows_that_fit(int64_t S, int64_t avail, F bytes)
{
    const int64_t q = dsai::kQueriesPerBlock;
    int64_t lo = 0, hi = S;  // bytes(lo) fits (or lo = 0), find the largest
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if (bytes(mid) <= avail) lo = mid; else hi = mid - 1;
    }
    return lo >= q || lo == S ? (lo == S ? lo : lo / q * q) : 0;
}

// fit_bytes > 0: the workspace is a fixed buffer of that many bytes (the
// no-allocation entry point); the launches are sized to fit it -- the
// few-query path in passes of the rows it holds, else streaming launches of
// the rows it holds -- and a problem that fits neither way is refused.
int score_topk_impl(indexer_t h, const void *q, const float *q_scale, const float *w,
                    int64_t w_stride_s, const void *k, const float *k_scale, int64_t S, int64_t T,
                    int H, int d, int m, int topk, int causal, int64_t q_pos0, const Docs &docs,
                    int32_t *idx, int32_t *valid_len, float *sel_score, void *workspace,
                    size_t workspace_bytes, void *stream, int64_t fit_bytes = 0,
                    const Witness &wit = Witness{})
{
    if (!h) return IDX_EINVAL;
    if (wit.n < 0 || (wit.n > 0 && (!wit.ptr || wit.stride < wit.n || !aligned(wit.ptr, 4))))
        return IDX_EINVAL;
    const indexer_config &cfg = h->cfg;
    const int flags = cfg.flags;
    const bool expand = flags & IDX_EXPAND, tail = flags & IDX_TAIL;
    // ---- sizes and modes
    if (S < 0 || T < 0 || H < 1 || d < 1 || m < 1 || topk < 1 || q_pos0 < 0) return IDX_EINVAL;
    if (causal != 0 && causal != 1) return IDX_EINVAL;
    if (w_stride_s != 0 && w_stride_s < H) return IDX_EINVAL;
    if (expand && topk % m) return IDX_EINVAL;
    if (tail && !causal) return IDX_EINVAL;
    if (tail && !docs.on && T < (q_pos0 + S) / m) return IDX_EINVAL;
    if (docs.on && (docs.ndoc < 0 || (docs.ndoc > 0 && (!docs.cu_q || !docs.cu_k)) ||
                    (docs.ndoc > 0 && expand && !docs.cu_tok)))
        return IDX_EINVAL;
    int W = 0;
    if (indexer_output_width(topk, m, flags, &W) != IDX_OK) return IDX_EINVAL;
    if (!shape_supported(cfg.dtype, H, d)) return IDX_EUNSUPPORTED;
    const int64_t ksel = ksel_of(topk, m, flags);
    if (ksel > kMaxSel) return IDX_EUNSUPPORTED;
    if (T >= INT32_MAX || (expand && T * (int64_t)m >= INT32_MAX) ||
        (tail && q_pos0 + S >= INT32_MAX))
        return IDX_EUNSUPPORTED;
    if (S == 0) return IDX_OK;
    // ---- pointers
    const bool fp8 = cfg.dtype == IDX_FP8_E4M3;
    if (!q || !w || !idx || !valid_len) return IDX_EINVAL;
    if (T > 0 && !k) return IDX_EINVAL;
    if (fp8 && (!q_scale || (T > 0 && !k_scale))) return IDX_EINVAL;
    if (!fp8 && (q_scale || k_scale)) return IDX_EINVAL;
    if (!aligned(q, 16) || (k && !aligned(k, 16)) || !aligned(w, 4)) return IDX_EINVAL;
    // ---- workspace
    const int64_t pmax = causal && !docs.on ? std::min<int64_t>(T, (q_pos0 + S) / m) : T;
    const int64_t cap = capacity(ksel, pmax);
    int64_t rows = rows_per_launch(cfg, S, capacity(ksel, T));
    const int64_t Tk = docs.on ? docs.row_keys : T;  // keys per few-query row
    bool few = use_few(cfg, S, Tk, ksel, docs.on ? docs.ndoc : -1);
    int64_t few_R = few ? few_rows(S, Tk, ksel) : 0;  // rows per few-query pass
    bool screen = !docs.on && !few && use_screen(cfg, H);
    size_t need =
        few     ? (size_t)FewLayout(few_R, Tk, ksel).bytes
        : docs.on ? (size_t)(rows * cap * (int64_t)sizeof(uint2))
                  : (size_t)workspace_need(cfg, S, T, H, ksel, pmax);
    if (fit_bytes > 0) {
        if (few) {
            few_R = std::min(few_R, rows_that_fit(S, fit_bytes, [&](int64_t r) {
                                   return FewLayout(r, Tk, ksel).bytes;
                               }));
            if (few_R < 1) few_R = 0, few = false;
        }
        screen = !docs.on && !few && use_screen(cfg, H);
        if (!few) {
            const bool scr = screen;
            rows = std::min(rows, rows_that_fit(S, fit_bytes, [&](int64_t r) {
                                return StreamLayout(r, cap, T, scr).bytes;
                            }));
            if (rows < 1) {
                g_detail = "the problem needs more scratch than the library's static " +
                           std::to_string(fit_bytes >> 20) + " MiB hold";
                return IDX_EWORKSPACE;
            }
        }
        need = few ? (size_t)FewLayout(few_R, Tk, ksel).bytes
                     : (size_t)StreamLayout(rows, cap, T, screen).bytes;
    }
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return IDX_EWORKSPACE;

    DeviceGuard guard(h->device);
    if (guard.err != hipSuccess) return fail_hip(guard.err);

    dsai::ScoreSelectParams p{};
    p.q = q;
    p.q_scale = q_scale;
    p.w = w;
    p.w_stride = w_stride_s;
    p.k = k;
    p.k_scale = k_scale;
    p.T = T;
    p.H = H;
    p.m = m;
    p.ksel = (int)ksel;
    p.causal = causal;
    p.expand = expand;
    p.tail = tail;
    p.q_pos0 = q_pos0;
    p.W = W;
    p.idx = idx;
    p.valid_len = valid_len;
    p.sel_score = sel_score;
    p.ws = static_cast<uint2 *>(workspace);
    p.cap = (int)cap;
    p.nsplit = 1;
    p.split_keys = round_up(std::max<int64_t>(T, 1), dsai::kKeysPerTile);
    p.cu_q = docs.cu_q;
    p.cu_k = docs.cu_k;
    p.pos0 = docs.pos0;
    p.cu_tok = docs.cu_tok;
    p.ndoc = docs.ndoc;
    p.varlen = docs.on;
    const int nb = (H + 31) / 32;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // element type the scoring kernels take: e4m3 on the fp8 MFMA when asked
    // for (d = 64, 128, unscreened), else the handle's dtype
    const int kdt = cfg.dtype == IDX_FP8_E4M3 && (flags & IDX_FP8_MFMA) && !screen &&
                            (d == 64 || d == 128)
                        ? 3 : cfg.dtype;
    if (few) {
        // Few-query path, in equal passes of at most the R rows the workspace
        // holds: all CUs score a sample of each row's keys; one block per
        // row cuts a threshold estimate from it; all CUs score the rows'
        // keys again and append only the keys at or above the estimate; one
        // block per row cuts the exact selection from those candidates and
        // writes the row, or marks it when they cannot hold the selection;
        // the streaming kernel then selects the marked rows (a launch whose
        // blocks return at once when no row of theirs is marked).
        const int64_t R = few_R;
        const FewLayout L(R, Tk, ksel);
        const int64_t npass = (S + R - 1) / R;
        const int64_t Rp = npass > 0 ? (S + npass - 1) / npass : R;
        char *base = static_cast<char *>(workspace);
        p.samp = reinterpret_cast<float *>(base);
        p.est = reinterpret_cast<uint32_t *>(base + L.est);
        p.fq_cnt = reinterpret_cast<uint32_t *>(base + L.cnt);
        p.status = reinterpret_cast<int32_t *>(base + L.stat);
        p.fq_dir = reinterpret_cast<uint2 *>(base + L.dir);
        p.ws = reinterpret_cast<uint2 *>(base + L.cand);
        p.cap = (int)L.cap;
        p.nbatch = L.nbatch;
        p.row_keys = Tk;
        p.split_keys = round_up(std::max<int64_t>(T, 1), dsai::kFewBatch);
        if (wit.n > 0 && !docs.on) {
            p.witness = wit.ptr;
            p.wit_stride = wit.stride;
            p.nwit = wit.n;
        }
        for (int64_t r0 = 0; r0 < S; r0 += Rp) {
            p.row0 = r0;
            p.nrows = std::min(Rp, S - r0);
            const int64_t groups = (p.nrows + dsai::kQueriesPerBlock - 1) / dsai::kQueriesPerBlock;
            const int64_t pm = causal && !docs.on
                                   ? std::min<int64_t>(T, (q_pos0 + r0 + p.nrows) / m) : T;
            const int64_t tiles = (std::max<int64_t>(pm, 1) + dsai::kKeysPerTile - 1) /
                                  dsai::kKeysPerTile;
            const int64_t want = std::max<int64_t>(1, (kFillBlocks + groups - 1) / groups);
            int64_t tiles_per = (tiles + std::min(want, tiles) - 1) / std::min(want, tiles);
            tiles_per = round_up(tiles_per, dsai::kFewBatch / dsai::kKeysPerTile);  // whole batches
            bool supported = true;
            hipError_t e = dsai::launch_score_rows(kdt, nb, d, docs.on, true, p, st,
                                                   &supported);
            if (!supported) return IDX_EUNSUPPORTED;
            if (e != hipSuccess) return fail_hip(e);
            e = dsai::launch_few_estimate(p, st);
            if (e != hipSuccess) return fail_hip(e);
            // one or two rows, or packed documents (each row its own key
            // window): the rows kernel; else query groups x key ranges
            p.split_keys = tiles_per * dsai::kKeysPerTile;
            p.nsplit = (int)((tiles + tiles_per - 1) / tiles_per);
            e = p.nrows <= kRowsKernelMax || docs.on
                    ? dsai::launch_score_rows(kdt, nb, d, docs.on, false, p, st, &supported)
                    : dsai::launch_score_select(kdt, nb, d, true, false, false, p, st,
                                                &supported);
            if (!supported) return IDX_EUNSUPPORTED;
            if (e != hipSuccess) return fail_hip(e);
            e = dsai::launch_few_finish(p, st);
            if (e != hipSuccess) return fail_hip(e);
            // repair: the marked rows through the streaming selection
            dsai::ScoreSelectParams pr = p;
            pr.repair = p.status;
            pr.nsplit = 1;
            pr.split_keys = round_up(std::max<int64_t>(T, 1), dsai::kFewBatch);
            e = dsai::launch_score_select(kdt, nb, d, false, docs.on, false, pr, st,
                                          &supported);
            if (!supported) return IDX_EUNSUPPORTED;
            if (e != hipSuccess) return fail_hip(e);
        }
        return IDX_OK;
    }
    if (screen) {
        // DoSA screening: key norms once, certificates per launch
        const StreamLayout L(rows, cap, T, true);
        char *base = static_cast<char *>(workspace);
        p.scr_stats = reinterpret_cast<unsigned long long *>(base);
        p.ws = reinterpret_cast<uint2 *>(base + L.cand);
        p.cert_perm = reinterpret_cast<int32_t *>(base + L.perm);
        p.cert_w = reinterpret_cast<float *>(base + L.w);
        p.cert_wt = reinterpret_cast<float *>(base + L.wt);
        p.cert_e = reinterpret_cast<float *>(base + L.e);
        p.cert_agg = reinterpret_cast<float *>(base + L.agg);
        p.knorm = reinterpret_cast<float *>(base + L.knorm);
        bool supported = true;
        const hipError_t e = dsai::launch_key_norms(cfg.dtype, d, p, st, &supported);
        if (!supported) return IDX_EUNSUPPORTED;
        if (e != hipSuccess) return fail_hip(e);
    }
    for (int64_t r0 = 0; r0 < S; r0 += rows) {
        p.row0 = r0;
        p.nrows = std::min(rows, S - r0);
        bool supported = true;
        hipError_t e = hipSuccess;
        if (screen) {
            // the certificate buffers hold one launch's rows
            e = dsai::launch_certificates(cfg.dtype, d, p, st, &supported);
            if (!supported) return IDX_EUNSUPPORTED;
            if (e != hipSuccess) return fail_hip(e);
        }
        e = dsai::launch_score_select(kdt, nb, d, false, docs.on, screen, p, st, &supported);
        if (!supported) return IDX_EUNSUPPORTED;
        if (e != hipSuccess) return fail_hip(e);
    }
    return IDX_OK;
}

}  // namespace

extern "C" {

int indexer_score_topk(indexer_t h, const void *q, const float *q_scale, const float *w,
                       int64_t w_stride_s, const void *k, const float *k_scale, int64_t S,
                       int64_t T, int H, int d, int m, int topk, int causal, int64_t q_pos0,
                       int32_t *idx, int32_t *valid_len, float *sel_score, void *workspace,
                       size_t workspace_bytes, void *stream)
{
    return score_topk_impl(h, q, q_scale, w, w_stride_s, k, k_scale, S, T, H, d, m, topk, causal,
                           q_pos0, Docs{}, idx, valid_len, sel_score, workspace, workspace_bytes,
                           stream);
}

int indexer_score_topk_witness(indexer_t h, const void *q, const float *q_scale, const float *w,
                               int64_t w_stride_s, const void *k, const float *k_scale,
                               int64_t S, int64_t T, int H, int d, int m, int topk, int causal,
                               int64_t q_pos0, const int32_t *witness, int64_t witness_stride,
                               int nwit, int32_t *idx, int32_t *valid_len, float *sel_score,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    Witness wit;
    wit.ptr = witness;
    wit.stride = witness_stride;
    wit.n = nwit;
    return score_topk_impl(h, q, q_scale, w, w_stride_s, k, k_scale, S, T, H, d, m, topk, causal,
                           q_pos0, Docs{}, idx, valid_len, sel_score, workspace, workspace_bytes,
                           stream, 0, wit);
}

int indexer_score_topk_noalloc(indexer_t h, const void *q, const float *q_scale, const float *w,
                               int64_t w_stride_s, const void *k, const float *k_scale,
                               int64_t S, int64_t T, int H, int d, int m, int topk, int causal,
                               int64_t q_pos0, int32_t *idx, int32_t *valid_len,
                               float *sel_score, void *stream)
{
    if (!h) return IDX_EINVAL;
    g_detail.clear();
    // Sizes that cannot fit are refused on the host before any HIP call: a
    // dry run of the sizing against a null workspace of the scratch's size
    // returns IDX_EWORKSPACE for "does not fit" and the validation codes for
    // bad arguments; only IDX_EWORKSPACE from a null workspace means "fits".
    const int64_t cap_bytes = (int64_t)dsai::noalloc_scratch_bytes();
    int rc = score_topk_impl(h, q, q_scale, w, w_stride_s, k, k_scale, S, T, H, d, m, topk,
                             causal, q_pos0, Docs{}, idx, valid_len, sel_score, nullptr,
                             (size_t)cap_bytes, stream, cap_bytes);
    if (rc != IDX_EWORKSPACE || !g_detail.empty()) return rc;  // invalid, S = 0, or too large
    DeviceGuard guard(h->device);
    if (guard.err != hipSuccess) return fail_hip(guard.err);
    void *scratch = nullptr;
    const hipError_t e = dsai::noalloc_scratch(h->device, &scratch);
    if (e != hipSuccess) return fail_hip(e);
    return score_topk_impl(h, q, q_scale, w, w_stride_s, k, k_scale, S, T, H, d, m, topk, causal,
                           q_pos0, Docs{}, idx, valid_len, sel_score, scratch, (size_t)cap_bytes,
                           stream, cap_bytes);
}

int indexer_workspace_bytes_varlen(indexer_t h, int64_t S, int64_t T, int H, int d, int m,
                                   int topk, int ndoc, int64_t max_doc_keys, size_t *bytes)
{
    if (!h || !bytes || S < 0 || T < 0 || H < 1 || d < 1 || m < 1 || topk < 1 || ndoc < 0 ||
        max_doc_keys < 0)
        return IDX_EINVAL;
    if ((h->cfg.flags & IDX_EXPAND) && topk % m) return IDX_EINVAL;
    const int64_t ksel = ksel_of(topk, m, h->cfg.flags);
    if (ksel > kMaxSel) return IDX_EUNSUPPORTED;
    const int64_t stream_bytes = rows_per_launch(h->cfg, S, capacity(ksel, T)) *
                                 capacity(ksel, T) * 8;
    const int64_t Tk = doc_row_keys(max_doc_keys, T);
    *bytes = (size_t)(use_few(h->cfg, S, Tk, ksel, ndoc) ? FewLayout(few_rows(S, Tk, ksel), Tk, ksel).bytes
                                                      : stream_bytes);
    return IDX_OK;
}

int indexer_score_topk_varlen(indexer_t h, const void *q, const float *q_scale, const float *w,
                              int64_t w_stride_s, const void *k, const float *k_scale, int64_t S,
                              int64_t T, int H, int d, int m, int topk, int causal,
                              const int32_t *cu_q, const int32_t *cu_k, const int64_t *pos0,
                              const int32_t *cu_tok, int ndoc, int64_t max_doc_keys,
                              int32_t *idx, int32_t *valid_len, float *sel_score,
                              void *workspace, size_t workspace_bytes, void *stream)
{
    if (max_doc_keys < 0) return IDX_EINVAL;
    Docs docs;
    docs.on = true;
    docs.cu_q = cu_q;
    docs.cu_k = cu_k;
    docs.pos0 = pos0;
    docs.cu_tok = cu_tok;
    docs.ndoc = ndoc;
    docs.row_keys = doc_row_keys(max_doc_keys, T);
    return score_topk_impl(h, q, q_scale, w, w_stride_s, k, k_scale, S, T, H, d, m, topk, causal,
                           0, docs, idx, valid_len, sel_score, workspace, workspace_bytes, stream);
}

int indexer_pair_regions(const int32_t *idx, const int32_t *valid_len, int64_t S, int W,
                         int32_t *shared, int32_t *left, int32_t *right, int32_t *counts,
                         void *stream)
{
    if (S < 0 || W < 1) return IDX_EINVAL;
    const int64_t npairs = S / 2;
    if (npairs == 0) return IDX_OK;
    if (!idx || !valid_len || !shared || !left || !right || !counts) return IDX_EINVAL;
    hipError_t e = dsai::launch_pair_regions(idx, valid_len, npairs, W, shared, left, right,
                                             counts, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? IDX_OK : fail_hip(e);
}

int indexer_pair_overlap(const int32_t *idx, const int32_t *valid_len, int64_t S, int W,
                         int32_t *shared, void *stream)
{
    if (S < 0 || W < 1) return IDX_EINVAL;
    const int64_t npairs = S / 2;
    if (npairs == 0) return IDX_OK;
    if (!idx || !valid_len || !shared) return IDX_EINVAL;
    hipError_t e = dsai::launch_pair_overlap(idx, valid_len, npairs, W, shared,
                                             static_cast<hipStream_t>(stream));
    return e == hipSuccess ? IDX_OK : fail_hip(e);
}

int indexer_overlap_summary(const int32_t *shared, const int32_t *valid_len, int64_t S,
                            indexer_overlap_stats *out)
{
    if (!out || S < 0) return IDX_EINVAL;
    const int64_t npairs = S / 2;
    if (npairs > 0 && (!shared || !valid_len)) return IDX_EINVAL;
    std::memset(out, 0, sizeof(*out));
    std::vector<double> ov;
    ov.reserve((size_t)npairs);
    double sum_ov = 0, sum_jac = 0, sum_sh = 0;
    int64_t ge50 = 0, ge75 = 0, ge80 = 0;
    for (int64_t i = 0; i < npairs; ++i) {
        const double va = valid_len[2 * i], vb = valid_len[2 * i + 1], sh = shared[i];
        if (std::min(va, vb) <= 0) {
            ++out->excluded;
            continue;
        }
        const double o = sh / std::min(va, vb);
        ov.push_back(o);
        sum_ov += o;
        sum_jac += sh / (va + vb - sh);
        sum_sh += sh;
        ge50 += o >= 0.5;
        ge75 += o >= 0.75;
        ge80 += o >= 0.8;
    }
    const int64_t n = (int64_t)ov.size();
    out->pairs = n;
    if (n == 0) return IDX_OK;
    std::sort(ov.begin(), ov.end());
    auto quantile = [&](double qq) {
        const double pos = qq * (double)(n - 1);
        const int64_t lo = (int64_t)std::floor(pos);
        const int64_t hi = std::min<int64_t>(lo + 1, n - 1);
        return ov[lo] + (pos - (double)lo) * (ov[hi] - ov[lo]);
    };
    out->mean_overlap = sum_ov / n;
    out->median_overlap = quantile(0.5);
    out->p90_overlap = quantile(0.9);
    out->mean_jaccard = sum_jac / n;
    out->mean_shared = sum_sh / n;
    out->frac_ge_50 = (double)ge50 / n;
    out->frac_ge_75 = (double)ge75 / n;
    out->frac_ge_80 = (double)ge80 / n;
    return IDX_OK;
}

#ifndef DSAI_SOURCE_HASH
#define DSAI_SOURCE_HASH "unknown"
#endif
const char *indexer_source_hash(void) { return DSAI_SOURCE_HASH; }

const char *indexer_strerror(int code)
{
    const char *base = "unknown status";
    switch (code) {
    case IDX_OK: base = "ok"; break;
    case IDX_EINVAL: base = "invalid argument"; break;
    case IDX_EUNSUPPORTED: base = "unsupported shape or dtype"; break;
    case IDX_EWORKSPACE: base = "workspace missing or too small"; break;
    case IDX_EHIP: base = "HIP error"; break;
    }
    if (code == IDX_EHIP && !g_hip_error.empty()) {
        g_msg = std::string(base) + ": " + g_hip_error;
        return g_msg.c_str();
    }
    if (code == IDX_EWORKSPACE && !g_detail.empty()) {
        g_msg = std::string(base) + ": " + g_detail;
        return g_msg.c_str();
    }
    return base;
}

}  // extern "C"

extern "C" int indexer_screen_certificates(indexer_t h, const void *q, const float *q_scale,
                                           const float *w, int64_t w_stride_s, int64_t S, int H,
                                           int d, const void *k, int64_t T, int m, int causal,
                                           int64_t q_pos0, int32_t *perm, float *weights,
                                           float *bound_weights, float *knorm_coef,
                                           float *aggregate, int32_t *activations, void *stream)
{
    if (!h || S < 0 || H < 1 || d < 1 || T < 0 || m < 1 || q_pos0 < 0) return IDX_EINVAL;
    if (causal != 0 && causal != 1) return IDX_EINVAL;
    if (w_stride_s != 0 && w_stride_s < H) return IDX_EINVAL;
    if (!shape_supported(h->cfg.dtype, H, d) || H <= 32 || H > 64) return IDX_EUNSUPPORTED;
    if (S == 0) return IDX_OK;
    const bool fp8 = h->cfg.dtype == IDX_FP8_E4M3;
    if (!q || !w || !perm || !weights || !bound_weights || !knorm_coef || !aggregate)
        return IDX_EINVAL;
    if (T > 0 && !k) return IDX_EINVAL;
    if (fp8 != (q_scale != nullptr)) return IDX_EINVAL;
    if (!aligned(q, 16) || (k && !aligned(k, 16)) || !aligned(w, 4)) return IDX_EINVAL;
    DeviceGuard guard(h->device);
    if (guard.err != hipSuccess) return fail_hip(guard.err);
    dsai::ScoreSelectParams p{};
    p.q = q;
    p.q_scale = q_scale;
    p.w = w;
    p.w_stride = w_stride_s;
    p.k = k;
    p.T = T;
    p.m = m;
    p.causal = causal;
    p.q_pos0 = q_pos0;
    p.H = H;
    p.row0 = 0;
    p.nrows = S;
    p.cert_perm = perm;
    p.cert_w = weights;
    p.cert_wt = bound_weights;
    p.cert_e = knorm_coef;
    p.cert_agg = aggregate;
    p.cert_act = activations;
    bool supported = true;
    const hipError_t e =
        dsai::launch_certificates(h->cfg.dtype, d, p, static_cast<hipStream_t>(stream), &supported);
    if (!supported) return IDX_EUNSUPPORTED;
    return e == hipSuccess ? IDX_OK : fail_hip(e);
}
