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
    // Dense mode (few queries): scores of each row's visible keys are written
    // to scores[row * sstride + key] instead of being selected in the kernel.
    float *scores;
    int64_t sstride;
    int nsplit;             // key ranges per query group; grid = groups * nsplit
    int64_t split_keys;     // keys per range, a multiple of kKeysPerTile
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
    // Few-query selection scratch (dense mode): per-row threshold estimate,
    // per (row, segment of dense_segment_keys() keys) candidate counts and
    // candidates as (score bits, key) (nseg segments per row,
    // dense_segment_keys() slots each).
    uint32_t *est;
    int32_t *seg_cnt;
    uint2 *seg_buf;
    int nseg;
    // Screening (DoSA certificates), per row of the launch: head order with
    // the kept heads first [nrows, 64] (-1 = no head), weights w * q_scale in
    // that order [nrows, 64], folded bound weights of the kept heads
    // [nrows, 32], key-norm coefficient [nrows]; key norms ||k_j|| [T].
    int32_t *cert_perm;
    float *cert_w;
    float *cert_wt;
    float *cert_e;
    float *knorm;
};

constexpr int kQueriesPerBlock = 8;   // one query per wave, 8 waves
constexpr int kKeysPerTile = 128;     // keys staged in LDS per step
constexpr int kSelGroup = 64;         // keys appended per selection step (one per lane)

// dtype codes match enum idx_dtype; dense = write scores (p.scores) instead
// of selecting; varlen = rows and keys are packed documents (p.cu_q ...)
hipError_t launch_score_select(int dtype, int nb, int d, bool dense, bool varlen, bool screen,
                               const ScoreSelectParams &p, hipStream_t stream, bool *supported);

// DoSA certificates of rows [p.row0, p.row0 + p.nrows) into p.cert_* (one
// wave per row), and the key norms p.knorm of all T keys.
hipError_t launch_certificates(int dtype, int d, const ScoreSelectParams &p, hipStream_t stream,
                               bool *supported);
hipError_t launch_key_norms(int dtype, int d, const ScoreSelectParams &p, hipStream_t stream,
                            bool *supported);

// Dense scores of one or two rows (p.scores, as the dense mode of
// launch_score_select writes them, bit for bit), every CU streaming its own
// slice of the keys; varlen: any number of packed-document rows, one per
// slab, each row's scores over its own key window.
hipError_t launch_score_rows(int dtype, int nb, int d, bool varlen, const ScoreSelectParams &p,
                             hipStream_t stream, bool *supported);

// Exact top-k of each row's dense scores and its canonical output row:
// threshold estimate per row, candidate filter per (row, key chunk), exact
// cut and output per row.
hipError_t launch_select_dense(const ScoreSelectParams &p, hipStream_t stream);
int dense_segment_keys();

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
