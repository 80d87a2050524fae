// Launch interface between the host C-ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsai {

// One launch of score_select covers `nrows` consecutive query rows.
struct ScoreSelectParams {
    const void *q;          // [S, H, d] codes (row-major)
    const float *q_scale;   // [S, H] or null
    const float *w;         // head weights, row t at w + t * w_stride
    int64_t w_stride;
    const void *k;          // [T, d] codes
    const float *k_scale;   // [T] or null
    int64_t row0;           // first row of this launch (row index within the call)
    int64_t nrows;          // rows in this launch
    int64_t T;
    int H;
    int m;                  // tokens per key
    int ksel;               // keys to select per query
    int causal;
    int expand;             // 1: key j -> positions j*m .. j*m+m-1
    int tail;               // 1: append positions P*m .. p
    int64_t q_pos0;
    int W;                  // output row width
    int32_t *idx;           // [S, W]
    int32_t *valid_len;     // [S]
    float *sel_score;       // [S, W] or null
    uint2 *ws;              // candidate buffers, [nrows, cap] of (score bits, key)
    int cap;                // candidate slots per query
    // Few-query mode (decode, small batches): the rows' keys are split over
    // all CUs; every key is scored once and only the (score bits, key) pairs
    // at or above the row's threshold estimate are appended to the row's
    // candidates ws[row * cap ...], one contiguous run per batch of kFewBatch
    // keys: batch b goes to sub-list b % kFewSub (kFewSubCap slots at
    // (b % kFewSub) * kFewSubCap), reserved with one atomic on that
    // sub-list's count fq_cnt[row * kFewSub + b % kFewSub] -- so concurrent
    // appends of one row spread over kFewSub counters; fq_dir[row * nbatch +
    // b] = (offset in the sub-list, count) of batch b.
    // samp[row * kSampStride ...] holds the exact scores of a key sample
    // from which est[row] is estimated, then of the row's witness keys;
    // status[row] = 1 leaves the row to the streaming kernel (repair).
    // row_keys bounds the keys of a row (packed documents: the caller's
    // max_doc_keys); nbatch = its batches.
    // witness (or null): row t's entries at witness + t * wit_stride, the
    // first nwit (at most kWitnessMax) of them scored: output indices of an
    // earlier selection (positions when expanding, else keys; -1 = none);
    // an entry names key e / m when expanding and e % m == 0, else key e,
    // and counts when that key is visible to the row.
    float *samp;
    const int32_t *witness;
    int64_t wit_stride;
    int nwit;
    uint32_t *est;
    uint32_t *fq_cnt;
    uint2 *fq_dir;
    int32_t *status;
    int64_t row_keys;
    int64_t nbatch;
    // Streaming kernel: when non-null, only rows with repair[row] != 0 are
    // scored and written (the few-query path's rows whose estimate failed).
    const int32_t *repair;
    int nsplit;             // key ranges per query group; grid = groups * nsplit
    int64_t split_keys;     // keys per range, a multiple of kFewBatch
    // Packed documents (varlen): rows [cu_q[i], cu_q[i+1]) are document i,
    // whose keys are k[cu_k[i], cu_k[i+1]); pos0[i] (or 0) is the position of
    // its first row within the document; expanded outputs are cu_tok[i] +
    // position.  Rows from cu_q[ndoc] on are padding.
    const int32_t *cu_q;
    const int32_t *cu_k;
    const int64_t *pos0;
    const int32_t *cu_tok;
    int ndoc;
    int varlen;             // 1: rows are packed documents (the fields above)
    // Screening (DoSA certificates), per row of the launch: head order with
    // the kept heads first [nrows, 64] (-1 = no head, kAggSlot = the
    // aggregate row, always slot 31 when present), weights w * q_scale in
    // that order [nrows, 64], folded bound weights of the kept heads
    // [nrows, 32], key-norm coefficient [nrows]; key norms ||k_j|| [T].
    int32_t *cert_perm;
    float *cert_w;
    float *cert_wt;
    float *cert_e;
    float *cert_agg;        // [nrows, d]: the aggregate row a~ (slot kAggSlot of the order)
    int32_t *cert_act;      // [nrows, 64] or null: seed activation counts (inspection)
    float *knorm;
    // screening statistics of the call (or null): keys tested against the
    // bound and keys that passed it; zeroed by the key-norm launch
    unsigned long long *scr_stats;
};

constexpr int kQueriesPerBlock = 8;   // one query per wave, 8 waves
constexpr int kKeysPerTile = 128;     // keys staged in LDS per step
constexpr int kSelGroup = 64;         // keys appended per selection step (one per lane)
constexpr int kAggSlot = -2;          // screening: head order entry of the aggregate row
constexpr int kFewBatch = 256;        // few-query: keys per candidate run (directory entry)
constexpr int kSampleKeys = 8192;     // few-query: keys in a row's estimate sample
constexpr int kFewCap = 8192;         // few-query: candidates the exact cut holds in LDS
constexpr int kFewSub = 32;           // few-query: candidate sub-lists per row (batch b: b % 32)
constexpr int kFewSubCap = 1024;      // few-query: entries per sub-list
constexpr int kWitnessMax = 8192;     // few-query: witness entries scored per row
constexpr int kSampStride = kSampleKeys + kWitnessMax;  // floats per row of samp

// dtype codes match enum idx_dtype, plus 3 = e4m3 on the fp8 MFMA (d = 64,
// 128; not screened); few = few-query mode (blocks over
// (query group, key range), candidates appended as described above) instead
// of selecting; varlen = rows and keys are packed documents (p.cu_q ...)
hipError_t launch_score_select(int dtype, int nb, int d, bool few, bool varlen, bool screen,
                               const ScoreSelectParams &p, hipStream_t stream, bool *supported);

// DoSA certificates of rows [p.row0, p.row0 + p.nrows) into p.cert_* (one
// wave per row), and the key norms p.knorm of all T keys.
hipError_t launch_certificates(int dtype, int d, const ScoreSelectParams &p, hipStream_t stream,
                               bool *supported);
hipError_t launch_key_norms(int dtype, int d, const ScoreSelectParams &p, hipStream_t stream,
                            bool *supported);

// Few-query scoring with q in registers and keys straight from memory,
// every CU streaming its own slice of the keys: sample = the exact scores of
// each row's key sample (p.samp); otherwise one or two rows (or, varlen, any
// number of packed-document rows, one per slab, each over its own key
// window) scored and filtered into candidates as the few-query mode of
// launch_score_select does, bit for bit.
hipError_t launch_score_rows(int dtype, int nb, int d, bool varlen, bool sample,
                             const ScoreSelectParams &p, hipStream_t stream, bool *supported);

// Few-query selection: the threshold estimate of each row from its sample
// (and the zeroing of its candidate count), before the filtering scoring
// launch; the exact cut and canonical output row of each row from its
// candidates (or status = 1 for the repair launch), after it.
hipError_t launch_few_estimate(const ScoreSelectParams &p, hipStream_t stream);
hipError_t launch_few_finish(const ScoreSelectParams &p, hipStream_t stream);

// Scratch of the no-allocation entry point: a static device array of
// noalloc_scratch_bytes() bytes per GPU; noalloc_scratch gives its device
// address on `device`, which must be the current device.
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(int device, void **ptr);

hipError_t launch_pair_overlap(const int32_t *idx, const int32_t *valid_len, int64_t npairs,
                               int W, int32_t *shared, hipStream_t stream);

hipError_t launch_pair_regions(const int32_t *idx, const int32_t *valid_len, int64_t npairs, int W,
                               int32_t *shared, int32_t *left, int32_t *right, int32_t *counts,
                               hipStream_t stream);

}  // namespace dsai
