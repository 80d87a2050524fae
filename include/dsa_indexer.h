/*
 * dsa_indexer.h -- C ABI of the MI355X (gfx950) lightning-indexer library.
 *
 * The operation (DoSA: Dots Sparse Attention, summary page, "Prerequisites:
 * DSA and the multi-head indexer"): for every query t and every key j that
 * t may see,
 *
 *     s_tj = sum_{h < H} w[t,h] * ReLU( q[t,h,:] . k[j,:] )
 *
 * with signed head weights w; then keep the top-k keys per query under one
 * total order -- higher score first, equal scores to the lower key index --
 * and hand them over sorted by KV index ("Adjacent-Query KV-Index Overlap in
 * 256K DSA Training", section 3: consumers read the canonical top-k indices
 * sorted by KV index).
 *
 * Keys may be tokens (m = 1) or m-token pools / compressed blocks (GLM-5.3-
 * Flash Module 06 "DSA & KPool"; the CSA abstract on the StreamIndex page).
 * Causality (Module 06, section 3): the query at absolute position p sees key
 * j iff (j+1)*m - 1 <= p, i.e. a pool becomes selectable once its last token
 * is visible.  Expansion and tail (Module 06, section 2): in expand mode each
 * selected pool becomes its m positions and the incomplete pool at the
 * query's own position (p+1 mod m positions, at most m-1) is appended as a
 * visible tail; rows are topk + m - 1 slots wide and padded.
 *
 * Memory: every pointer below is a caller-owned buffer.  Pointers documented
 * as "device" must point to device memory of the device the handle was
 * created for; "host" pointers to host memory.  The library never allocates
 * device memory: scratch space comes from the caller's workspace buffer.
 * Work is enqueued on the caller's HIP stream (hipStream_t passed as void*,
 * NULL = the default stream); no call synchronises with the host.
 *
 * Errors: every entry point returns IDX_OK (0) or a negative IDX_E* code.
 * Arguments are validated on the host before anything is enqueued, so a
 * failed validation leaves every output untouched.  A failed launch returns
 * IDX_EHIP; indexer_strerror() then also reports the HIP error text of the
 * calling thread's last failure.
 */
#ifndef DSA_INDEXER_H
#define DSA_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct indexer_s *indexer_t;

/* Element type of q and k.  FP8 is OCP e4m3 (e4m3fn: max 448, no inf). */
enum idx_dtype { IDX_F32 = 0, IDX_BF16 = 1, IDX_FP8_E4M3 = 2 };

/* Output mode flags. */
enum {
    IDX_EXPAND = 1, /* selected pools expand to their m token positions   */
    IDX_TAIL = 2,   /* append the incomplete pool (needs EXPAND, causal)  */
    IDX_SCREEN = 4, /* DoSA certificate screening, see below              */
    /* IDX_FP8_E4M3 only: contract the e4m3 codes as they are on the gfx950
     * fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) instead of widening them
     * exactly to bf16 for the bf16 MFMA.  Twice the matrix rate, but the
     * instruction sums its 64 products at reduced internal precision, so
     * scores differ from the fp32-accumulated ones by more than rounding
     * (within the fp8 tolerance of the scores the pages' systems compute
     * on fp8 tensor cores).  d in {64, 128}; ignored for d = 32 and with
     * IDX_SCREEN (whose bound needs fp32-accumulated products). */
    IDX_FP8_MFMA = 8
};

enum {
    IDX_OK = 0,
    IDX_EINVAL = -1,       /* bad argument (null pointer, size, flag mix) */
    IDX_EUNSUPPORTED = -2, /* valid but not built (H, d, dtype combination) */
    IDX_EWORKSPACE = -3,   /* workspace missing or smaller than required  */
    IDX_EHIP = -4          /* a HIP runtime call or launch failed         */
};

typedef struct {
    int dtype;           /* enum idx_dtype                                     */
    int flags;           /* IDX_EXPAND | IDX_TAIL | IDX_SCREEN | IDX_FP8_MFMA  */
    int64_t query_chunk; /* queries per streaming launch (bounds the workspace);
                          * 0 = as many as 4 GiB of candidate buffers hold
                          * (at least 2048); results do not depend on it    */
    /* Few-query path (decode, small batches against a long key set): when
     * S <= few_query_rows, all CUs score a sample of each row's keys (8,192
     * keys in 128 runs of 64), one block per row cuts a threshold estimate
     * from it, all CUs score the rows' keys and append only the (score, key)
     * pairs at or above the estimate to the row's candidate list (the DoSA
     * summary's sparse write-back: no score array is written), and one block
     * per row cuts the exact selection from its candidates; a row whose
     * candidates cannot hold the selection (the estimate too high, or more
     * than 8,192 candidates) is selected by a streaming launch over the
     * marked rows.  Otherwise rows are scored and selected in one streaming
     * pass per query chunk.  0 = default: 1024, or 64 for packed documents
     * with more than two rows per document (indexer_score_topk_varlen: S >
     * 2 ndoc), whose rows share key tiles on the streaming path; negative =
     * never.  Both paths give identical results.  The few-query workspace
     * holds, each part starting on a 256-byte boundary, the samples' and
     * witnesses' scores (S * 16384 * 4 bytes), the estimates (S * 4), the
     * candidate sub-list counts (S * 32 * 4), the repair marks (S * 4), a
     * directory of (offset, count) per 256 keys of a row (S * ceil(Tk /
     * 256) * 8; Tk = T, or max_doc_keys for packed documents) and the
     * candidate lists (S * cap * 8, cap = max(32768, the streaming path's
     * slots per row)) -- about 330 KB per row at 262,144 keys.  It is
     * capped at 4 GiB: when the S rows need more, it is sized for the R
     * rows that fit and the rows are taken in ceil(S / R) equal passes. */
    int64_t few_query_rows;
} indexer_config;

/* Limits of this build (IDX_EUNSUPPORTED outside them):
 *   1 <= H <= 64; d in {32, 64} (fp32), {32, 64, 128} (bf16, fp8);
 *   1 <= topk, selected keys per query (topk, or topk/m in expand mode)
 *   <= 16000; T < 2^31 keys; output positions < 2^31. */

/* Create a handle.  Host-only: records the configuration and device number;
 * makes no HIP call.  *out receives the handle (caller frees it with
 * indexer_destroy).  IDX_EINVAL on a null pointer or unknown dtype/flags. */
int indexer_create(const indexer_config *cfg, int device, indexer_t *out);

/* Release a handle (NULL is accepted). */
int indexer_destroy(indexer_t h);

/* Row width of idx / sel_score: topk + (m-1 if IDX_TAIL) -- 2,051 for
 * topk 2048, m 4 with the tail (Module 06, section 2).  Host-only. */
int indexer_output_width(int topk, int m, int flags, int *W);

/* Device workspace bytes that indexer_score_topk needs for this problem
 * with this handle: per-query candidate buffers for one query chunk, or the
 * few-query layout (samples, candidate lists, directory).  Host-only; depends on S,
 * query_chunk, few_query_rows, T, m, topk and the flags. */
int indexer_workspace_bytes(indexer_t h, int64_t S, int64_t T, int H, int d, int m, int topk,
                            size_t *bytes);

/*
 * Score every visible key for S queries and write each query's top-k.
 *
 *   q          device, [S, H, d] of cfg.dtype, row-major.
 *   q_scale    device, [S, H] fp32 per-row dequantisation scale (fp8 only;
 *              must be NULL for f32/bf16).  Dequantised q = code * scale.
 *   w          device, fp32; row t's head weights are w[t*w_stride_s + h]
 *              (w_stride_s = H for an [S, H] array, 0 to broadcast one [H]).
 *   k          device, [T, d] of cfg.dtype, row-major.
 *   k_scale    device, [T] fp32 (fp8 only, else NULL).
 *   S, T, H, d sizes (S = 0 or T = 0 are valid).
 *   m          tokens per key (1 = token keys).
 *   topk       output units per query: token positions in expand mode (must
 *              be a multiple of m; topk/m pools are selected), keys otherwise.
 *   causal     1: row t sits at absolute position p = q_pos0 + t and sees
 *              key j iff (j+1)*m - 1 <= p; 0: every key is visible.
 *   q_pos0     absolute position of row 0 (external chunking, decode).
 *   idx        device, [S, W] int32 out (W from indexer_output_width):
 *              ascending indices, then -1 padding.  Expand mode: token
 *              positions (tail positions last); otherwise key indices.
 *   valid_len  device, [S] int32 out: number of valid entries of each row =
 *              min(Ksel, P_t) * (m if expand) + tail, P_t visible keys.
 *   sel_score  device, [S, W] fp32 out or NULL: the fp32 score of the key
 *              behind each entry; 0 for tail and padding slots.  With NULL,
 *              rows that see at most Ksel keys (all of them selected) are
 *              answered without scoring on the streaming path.
 *   workspace  device, >= indexer_workspace_bytes(...) bytes, 16-B aligned;
 *              contents on entry are ignored, on return undefined.
 *   stream     hipStream_t (void*), NULL = default stream.
 *
 * IDX_TAIL requires IDX_EXPAND, causal = 1 and T >= (q_pos0 + S) / m (every
 * complete pool present), else IDX_EINVAL.  q and k must be 16-B aligned
 * (IDX_EINVAL).  Preconditions not checked on
 * the device: finite inputs, scales > 0, q/k/w/scale buffers as described.
 * Calls sharing one workspace must be ordered on one stream.
 */
int indexer_score_topk(indexer_t h, const void *q, const float *q_scale, const float *w,
                       int64_t w_stride_s, const void *k, const float *k_scale, int64_t S,
                       int64_t T, int H, int d, int m, int topk, int causal, int64_t q_pos0,
                       int32_t *idx, int32_t *valid_len, float *sel_score, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * indexer_score_topk with witness keys for the few-query path ("DoSA: Dots
 * Sparse Attention", summary page, "Method steps": decode scores every key
 * and takes keys selected at an earlier step as witnesses for a threshold
 * that cannot exceed the current one).  Same arguments, results and errors
 * as indexer_score_topk, plus:
 *   witness         device int32 [S, witness_stride], in: row t's entries
 *                   start at witness + t * witness_stride; the first
 *                   min(nwit, 8192) are used.  Each is an output index as
 *                   this handle writes them (a token position when
 *                   IDX_EXPAND is set, else a key index), typically the
 *                   row's idx of the previous decode step; -1 means none.
 *                   When expanding, an entry names key e / m if e % m == 0
 *                   (the first position of a pool) and nothing otherwise, so
 *                   a whole output row names each of its pools once; an
 *                   entry naming a key the row does not see is ignored.
 *   witness_stride  >= nwit (IDX_EINVAL otherwise); nwit >= 0, 0 = none.
 * Rows taken by the few-query path score their witness keys with the
 * sample; when the witnesses name at least Ksel visible keys, the Ksel-th
 * best of their exact scores replaces the sampled estimate if it is higher.
 * Distinct witnesses make it a lower bound of the row's Ksel-th best score,
 * so no key of the selection is filtered out; repeated ones can make it
 * too high, which the exact cut detects (the row then goes to the repair
 * launch).  The result is the exact selection in every case, identical to
 * indexer_score_topk's; witnesses change only the work.  The streaming path
 * (rows beyond the few-query limit) ignores them.
 */
int indexer_score_topk_witness(indexer_t h, const void *q, const float *q_scale, const float *w,
                               int64_t w_stride_s, const void *k, const float *k_scale,
                               int64_t S, int64_t T, int H, int d, int m, int topk, int causal,
                               int64_t q_pos0, const int32_t *witness, int64_t witness_stride,
                               int nwit, int32_t *idx, int32_t *valid_len, float *sel_score,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * indexer_score_topk without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Scratch space comes from a static
 * device array of the library, 256 MiB on every GPU the library runs on,
 * held until the process ends.  Arguments, results and errors are those of
 * indexer_score_topk (same kernels, bit-identical results); the launches
 * are sized to fit the array: the few-query path in passes of the rows it
 * holds when one row fits, else streaming launches of at most the rows it
 * holds (and at most query_chunk).  A problem that fits neither way (only
 * possible with IDX_SCREEN and more than about 66 million keys) returns
 * IDX_EWORKSPACE before any HIP call, and indexer_strerror names the limit.
 * No call allocates or frees memory.  Every call on one GPU uses that GPU's
 * array, so calls that may overlap on one GPU (several streams, or threads
 * without ordering) race and must be serialised by the caller.
 */
int indexer_score_topk_noalloc(indexer_t h, const void *q, const float *q_scale, const float *w,
                               int64_t w_stride_s, const void *k, const float *k_scale,
                               int64_t S, int64_t T, int H, int d, int m, int topk, int causal,
                               int64_t q_pos0, int32_t *idx, int32_t *valid_len,
                               float *sel_score, void *stream);

/*
 * Packed documents ("varlen"; GLM-5.3-Flash Module 06 "DSA & KPool", section
 * 3: a pool may not span a document boundary, and one document's tokens may
 * not influence another document's selection).  The same operation as
 * indexer_score_topk, per document: row t of document i sits at position
 * p = pos0[i] + (t - cu_q[i]) of that document and sees the document's keys
 * j (local index) with (j+1)*m - 1 <= p (causal) or all of them; pools are
 * the caller's per-document keys, so none spans a boundary.
 *
 *   cu_q    device int32 [ndoc + 1]: rows of document i are
 *           [cu_q[i], cu_q[i+1]); non-decreasing, cu_q[0] = 0,
 *           cu_q[ndoc] <= S.  Rows from cu_q[ndoc] on are padding: their
 *           output row is all -1 and valid_len 0.
 *   cu_k    device int32 [ndoc + 1]: keys of document i are
 *           k[cu_k[i], cu_k[i+1]); non-decreasing, cu_k[ndoc] <= T.
 *   pos0    device int64 [ndoc] or NULL (all 0): position within document i
 *           of its first row (a later prefill chunk, or one decode row per
 *           sequence at the end of its context).
 *   cu_tok  device int32 [ndoc], required with IDX_EXPAND: packed-token
 *           index of document i's position 0.
 *   max_doc_keys  host int64: an upper bound on every document's key count
 *           cu_k[i+1] - cu_k[i] (as a maximum sequence length is passed to
 *           varlen attention); 0 = unknown, taken as T; values above T are
 *           taken as T; negative: IDX_EINVAL.  It sizes the few-query
 *           path's per-row directory and candidate slots (by max_doc_keys
 *           keys instead of T), so batched decode over many documents needs
 *           far less workspace; the streaming path does not use it.  A
 *           document with more keys breaks the precondition: its rows'
 *           selection is then unspecified, but every access stays in bounds.
 *   Output entries: compressed keys as global key indices cu_k[i] + j;
 *   with IDX_EXPAND, token indices cu_tok[i] + position (pool j expands to
 *   positions j*m .. j*m+m-1; with IDX_TAIL the positions from P*m to p of
 *   the document's incomplete pool follow).
 *
 * Every other argument, the width W, the tie rule and the ordering are as
 * in indexer_score_topk (its q_pos0 has no counterpart here).  The offset
 * arrays are read on the device only, so their preconditions are not
 * checked on the host; offsets are clamped to [0, T], and a row whose
 * document lacks complete pools gets a tail clipped to the row width.  With
 * IDX_EXPAND the caller keeps every output index below 2^31.  With at most
 * few_query_rows rows (batched decode: one row per sequence) the rows take
 * the few-query path (each row's own key window, at most max_doc_keys keys,
 * scored by all CUs with only the keys at or above the row's estimate kept,
 * then the per-row exact cut; in equal passes when S rows need more than
 * 4 GiB); otherwise the streaming path.
 * With the default few_query_rows that means up to 1024 rows when S <= 2
 * ndoc, else up to 64.  Both give identical results.  Workspace from
 * indexer_workspace_bytes_varlen with the same S, T, ndoc and max_doc_keys.
 */
int indexer_score_topk_varlen(indexer_t h, const void *q, const float *q_scale, const float *w,
                              int64_t w_stride_s, const void *k, const float *k_scale, int64_t S,
                              int64_t T, int H, int d, int m, int topk, int causal,
                              const int32_t *cu_q, const int32_t *cu_k, const int64_t *pos0,
                              const int32_t *cu_tok, int ndoc, int64_t max_doc_keys,
                              int32_t *idx, int32_t *valid_len, float *sel_score,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Device workspace bytes for indexer_score_topk_varlen with the same S, T,
 * ndoc and max_doc_keys: the few-query layout of indexer_config.
 * few_query_rows for S rows of max_doc_keys keys (0: T) when that path is
 * taken, else candidate buffers for one query chunk of up to min(S,
 * query_chunk) rows (0: as for indexer_score_topk), each bounded by T keys.
 * Host-only. */
int indexer_workspace_bytes_varlen(indexer_t h, int64_t S, int64_t T, int H, int d, int m,
                                   int topk, int ndoc, int64_t max_doc_keys, size_t *bytes);

/*
 * Adjacent-pair overlap diagnostic ("Adjacent-Query KV-Index Overlap in
 * 256K DSA Training", sections 1 and 3): for each non-overlapping pair
 * (rows 2i, 2i+1), i < S/2, shared[i] = |A_2i ∩ A_2i+1| where A_t is
 * idx[t, 0:valid_len[t]] (ascending, as indexer_score_topk writes it);
 * exact intersection (a bitmap over the pair's index range in LDS), no
 * all-pairs comparison.
 *   idx [S, W] int32, valid_len [S] int32: device, in.
 *   shared [S/2] int32: device, out.  An odd last row is unpaired.
 */
int indexer_pair_overlap(const int32_t *idx, const int32_t *valid_len, int64_t S, int W,
                         int32_t *shared, void *stream);

/*
 * q-cluster preprocessing ("Adjacent-Query KV-Index Overlap in 256K DSA
 * Training", sections 6.1, 6.2 and 6.4): for each non-overlapping pair
 * (rows 2i, 2i+1), i < S/2, split the two index rows into the entries both
 * hold, the entries only row 2i holds and the entries only row 2i+1 holds.
 * The exact split is computed here (no fixed shared count is assumed), into
 * fixed-capacity buffers with device-side counts, so a captured launch
 * sequence stays valid whatever the overlap.
 *   idx [S, W] int32, valid_len [S] int32: device, in; each row's first
 *     valid_len entries ascending (as indexer_score_topk writes them).
 *   shared, left, right: device [S/2, W] int32, out: the region's entries
 *     ascending, then -1.
 *   counts: device [S/2, 3] int32, out: sizes of shared, left, right
 *     (shared + left = valid_len[2i], shared + right = valid_len[2i+1]).
 * An odd last row is unpaired.
 */
int indexer_pair_regions(const int32_t *idx, const int32_t *valid_len, int64_t S, int W,
                         int32_t *shared, int32_t *left, int32_t *right, int32_t *counts,
                         void *stream);

/* Summary of the adjacent-pair statistic over host copies of shared[S/2]
 * and valid_len[S].  Overlap of a pair = shared / min(vA, vB) (normalised by
 * the rows' valid top-k lengths); Jaccard = shared / (vA + vB - shared).
 * Pairs with an empty row are counted in `excluded` and left out.  Median
 * and P90 interpolate linearly between order statistics.  Host-only. */
typedef struct {
    int64_t pairs, excluded;
    double mean_overlap, median_overlap, p90_overlap, mean_jaccard, mean_shared;
    double frac_ge_50, frac_ge_75, frac_ge_80;
} indexer_overlap_stats;

int indexer_overlap_summary(const int32_t *shared, const int32_t *valid_len, int64_t S,
                            indexer_overlap_stats *out);

/* DoSA certificate screening ("DoSA: Dots Sparse Attention", summary page,
 * "Core method", "Method steps" and "Technical novelty").  With IDX_SCREEN
 * in the flags, the streaming path (not the few-query or packed-document
 * paths) with 33 <= H <= 64 first builds one certificate per query row from
 * its head codes q_h, weights a_h = w_h q_scale_h and a seed set of its
 * visible keys (256 keys spread evenly over them, or all of them):
 *  - each head's activation frequency p_h on the seeds (share with
 *    q_h . k > 0);
 *  - a head budget r = 31 when H <= 63 (the last row of the kept block then
 *    holds the aggregate below), else 32: all positive heads plus the
 *    negative heads of largest |a_h| ||q_h|| min(p_h, 1 - p_h) when at most
 *    r heads are positive, else the r positive heads of largest
 *    a_h ||q_h||;
 *  - each omitted positive head folded onto the kept positive head closest
 *    in direction, its residual bounded jointly over the omitted heads;
 *  - the omitted negative heads with p_h >= 1/2 summed into one aggregate
 *    row a_A = sum |a_h| q_h, whose ReLU(a_A . k) the bound subtracts;
 *  - a coefficient of ||k|| that holds the residual allowance, the
 *    aggregate's rounding and a margin for fp32 rounding.
 * Every key's upper bound U = sum_kept w~_h ReLU(q_h . k) - ReLU(a_A . k)
 * + coef ||k|| (times k_scale) comes from the kept block alone; a key with
 * U below the row's running Ksel-th score lower bound is not scored
 * further, the others get the remaining heads.  Lossless: the selection
 * equals the unscreened one up to the order in which the head terms are
 * summed (the kept heads come first).  The workspace grows by 1156 bytes
 * per row of a launch, 4 per key and 256 (indexer_workspace_bytes accounts
 * for it).  After a screened call (ordered on its stream) the workspace's
 * first 16 bytes hold two uint64 counts for the call: keys tested against
 * a bound, and keys whose bound reached the row's running threshold (and
 * got the remaining heads); the rest of the workspace stays undefined.
 *
 * indexer_screen_certificates writes the certificates of S rows as the
 * screened path uses them, for inspection:
 *   q, q_scale, w, w_stride: as for indexer_score_topk (device).
 *   k, T, m, causal, q_pos0: the keys the seeds come from and the rows'
 *     visibility, as for indexer_score_topk; k = NULL or T = 0 means no
 *     seeds: every p_h is taken as 1/2 and there is no aggregate.
 *   perm: device int32 [S, 64], out: head order, kept heads first (by head
 *     index), then at slot 31 the aggregate (-2) when there is one, then
 *     the omitted heads (by index), then -1.
 *   weights: device fp32 [S, 64], out: w_h * q_scale_h (w_h for bf16 and
 *     fp32) in that order; 0 for the aggregate.
 *   bound_weights: device fp32 [S, 32], out: the kept heads' folded weights
 *     (-1 for the aggregate).
 *   knorm_coef: device fp32 [S], out: the coefficient of ||k|| (raw codes).
 *   aggregate: device fp32 [S, d], out: a_A as the matrix unit reads it
 *     (rounded to bf16 except for fp32 data); written only for rows that
 *     have an aggregate.
 *   activations: device int32 [S, 64] or NULL, out: seed count with
 *     q_h . k > 0 per head (by head index; 0 past H).
 * Requires 33 <= H <= 64 (else IDX_EUNSUPPORTED).  Asynchronous on `stream`.
 */
int indexer_screen_certificates(indexer_t h, const void *q, const float *q_scale, const float *w,
                                int64_t w_stride, int64_t S, int H, int d, const void *k,
                                int64_t T, int m, int causal, int64_t q_pos0, int32_t *perm,
                                float *weights, float *bound_weights, float *knorm_coef,
                                float *aggregate, int32_t *activations, void *stream);

/* Static text for a status code, followed (for IDX_EHIP) by the calling
 * thread's last HIP error.  Never NULL. */
const char *indexer_strerror(int code);

/* Identification of the build: a short hash of the sources and compile
 * flags the library was built from ("unknown" if the build did not set it),
 * so a loader can refuse a library that no longer matches its sources.
 * Static string, never NULL. */
const char *indexer_source_hash(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_INDEXER_H */
