// score_select: fused lightning-indexer scoring + streaming top-k for gfx950.
//
// Computes, for each query row t and each visible key j,
//     s_tj = sum_h w[t,h] * ReLU(q[t,h,:] . k[j,:])
// (DoSA: Dots Sparse Attention, summary page, "Prerequisites": signed-ReLU
// multi-head indexer) and keeps the exact top-Ksel keys of each row under the
// total order (higher score, then lower index), without ever writing a score
// tensor: StreamIndex's point (abstract on the StreamIndex page) that the
// [S, H, T] or [S, T] intermediate never exists.
//
// Work decomposition (one block = 8 consecutive queries, one per wave):
//  * The block walks the keys visible to its last query in tiles of 128 keys.
//    Each tile is staged once into LDS (XOR-swizzled 16-B chunks, double
//    buffered: tile i+1 is fetched into registers while tile i is scored) and
//    read by all 8 waves, so every key row is fetched from L2 once per 8
//    queries.  Blocks are issued heaviest-first (last query group first) so
//    the causal triangle's long rows start early.
//  * A wave holds its query's q[t, :, :] in registers as MFMA A operands:
//    A rows = 32 heads per block (NB blocks cover H <= 32*NB heads; missing
//    heads are zero rows with zero weight), B columns = 32 keys, the d axis
//    is the contraction.  bf16: v_mfma_f32_32x32x16_bf16; fp8 (OCP e4m3):
//    codes widened exactly to bf16 in registers / while staging to LDS, then
//    the same bf16 MFMA (fp32 accumulation); fp32: v_mfma_f32_32x32x2_f32.
//    Accumulators hold 16 heads x 1 key per lane; the signed-ReLU head sum
//    runs in registers (max + fma per element), and a swap of register
//    halves between the two 16-head partial sums (v_permlane32_swap)
//    finishes it: each lane ends with the score of one key of a 64-key
//    selection group.
//  * The MFMAs of one (32-key column block, 32-head block) step are issued
//    interleaved with the epilogue of the previous step and with the LDS
//    reads of the next column block's B operands, so the VALU work runs in
//    the shadow of the matrix pipe instead of after it.
//  * fp8: per-row scales fold out of the ReLU because it is positively
//    homogeneous (DoSA summary, "ReLU subadditivity, positive homogeneity"):
//    w'[t,h] = w[t,h] * q_scale[t,h] multiplies the head sum, k_scale[j]
//    multiplies the finished score.
//  * The two waves that share a SIMD (w and w + 4) select at opposite ends of
//    a tile, so one wave's branchy selection overlaps the other's MFMAs; the
//    wave in its MFMA phase runs at raised issue priority (s_setprio).
//  * Optional screening (SCREEN instance; DoSA summary, "Method steps"):
//    head block 0 holds a per-row certificate's kept heads and bounds every
//    key; only keys whose bound reaches the running threshold get block 1,
//    gathered 32 per MFMA column block (see screen_tile below).
//
// Streaming selection (per wave, per query; no block barrier involved):
//  * Scores map to an order-preserving 32-bit code u (-0 folded into +0).
//  * tau is a running lower bound on the final Ksel-th code: any visible key
//    subset of size >= Ksel has a Ksel-th score no larger than the full set's
//    (DoSA summary, "Top-K threshold and subset lower bound").  Keys scan in
//    ascending index order, so a new key can only enter if u >= tau.
//    The pass test runs on the float score against the threshold's decoded
//    value, which is exactly equivalent to comparing codes.
//  * Survivors are appended, ballot-compacted, to the query's candidate buffer
//    in global memory (ascending key order is preserved), and counted in a
//    4096-bin LDS histogram of u's top 12 bits (16-bit packed counters).
//  * Once Ksel entries exist, the wave tracks the histogram bin tb holding
//    the Ksel-th best code and the count above it; when that count runs a
//    group past Ksel, tb advances (64 bins per lane-parallel step) and tau
//    rises to tb's lower edge.  Entries below tau are never appended.
//  * If the buffer could still overflow, the histogram gives a cut; entries
//    below it are dropped in one stable in-place pass.  Near-ties in one bin
//    are resolved by two more radix levels (10 + 10 bits), and equal codes
//    are cut by buffer position, which is key order -- the tie rule.
//  * After the last tile the exact selection runs once more (boundary-bin
//    codes gathered into the idle K tiles in LDS) and writes the output row
//    directly: survivors in buffer order are already sorted by KV index
//    ("Adjacent-Query KV-Index Overlap in 256K DSA Training", section 3),
//    pools expand to m positions and the incomplete tail follows
//    (GLM-5.3-Flash Module 06 "DSA & KPool", section 2), then -1 padding.
//  * A row that sees at most Ksel keys selects all of them whatever their
//    scores (valid_len = min(Ksel, visible)); when no selected scores are
//    asked for, a block whose rows all see at most Ksel keys loads and
//    scores nothing and writes those keys directly (the first Ksel*m
//    positions of a sequence, documents shorter than that).
#include "kernels.h"
#include "mfma_ops.h"
#include "select_common.h"

namespace dsai {
namespace {

constexpr int kThreads = kQueriesPerBlock * 64;

template <int DT, int NB, int D, bool FEW, bool VARLEN, bool SCREEN>
__global__ void __launch_bounds__(kThreads, 1) score_select_kernel(ScoreSelectParams p)
{
    static_assert(!SCREEN || (NB == 2 && !FEW && !VARLEN && DT != 3),
                  "screening: two head blocks, fp32-accumulated products");
    using O = Op<DT, D>;
    using A = typename O::A;
    constexpr int KS = O::KS, NCH = O::NCH, GCH = O::GCH, ES = O::ES, CPK = O::CPK;
    constexpr bool kScaled = DT >= 2;  // fp8 codes: per-row scales fold out of the ReLU
    constexpr int TILE_CH = kKeysPerTile * NCH;     // LDS 16-B chunks per tile
    constexpr int GTILE_CH = kKeysPerTile * GCH;    // global 16-B chunks per tile
    constexpr int CPT = (GTILE_CH + kThreads - 1) / kThreads;
    constexpr int SWZ = (NCH < 16 ? NCH : 16) - 1;
    constexpr int64_t ROWB = (int64_t)D * ES;

    __shared__ uint4 ktile[2][TILE_CH];
    __shared__ float kscale_tile[2][kKeysPerTile];
    __shared__ uint32_t hist_all[kQueriesPerBlock][kHistWords];
    // screening only: key norms of the staged tiles, each wave's kept-head
    // partial sums of one tile (two lane halves) and its survivor list
    constexpr int kScr = SCREEN ? 1 : 0;
    __shared__ float knorm_tile[2][kScr * kKeysPerTile + 1];
    __shared__ float p0_all[kQueriesPerBlock][kScr * 2 * kKeysPerTile + 1];
    __shared__ uint16_t sl_all[kQueriesPerBlock][kScr * kKeysPerTile + 1];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int hh = lane >> 5, l32 = lane & 31;
    const int64_t ngroups = (p.nrows + kQueriesPerBlock - 1) / kQueriesPerBlock;
    // few-query mode: block = (query group, key range); streaming: one range
    const int64_t gi = FEW ? (int64_t)blockIdx.x / p.nsplit : (int64_t)blockIdx.x;
    const int sp = FEW ? (int)((int64_t)blockIdx.x - gi * p.nsplit) : 0;
    const int64_t grp = ngroups - 1 - gi;  // heaviest rows first
    const int64_t qrow = grp * kQueriesPerBlock + wave;
    // repair launch (few-query rows whose estimate failed): only those rows
    // are scored and written; a block with none of them returns at once
    const bool active = qrow < p.nrows && (!p.repair || p.repair[qrow] != 0);
    if (!FEW && p.repair && !__syncthreads_or(active)) return;
    const int64_t t = p.row0 + qrow;
    // This row's key window [klo, klo + Pq) and the token position of its
    // key 0 (tok0, expanded outputs).  One document: every key from 0, the
    // row at position q_pos0 + t.  Packed documents: the row's document's
    // keys, its position inside that document.
    int64_t pos, Pq, klo = 0, tok0 = 0;
    int64_t kbeg, kend;  // keys this block walks
    int64_t Pmax;        // most keys any row of the block sees
    if constexpr (VARLEN) {
        __shared__ int64_t wlo[kQueriesPerBlock], whi[kQueriesPerBlock];
        const DocWindow dw = active ? doc_window(p, t) : DocWindow{};
        pos = dw.pos;
        Pq = dw.P;
        klo = dw.klo;
        tok0 = dw.tok0;
        if (lane == 0) {
            wlo[wave] = Pq > 0 ? klo : INT64_MAX;
            whi[wave] = Pq > 0 ? klo + Pq : INT64_MIN;
        }
        __syncthreads();
        kbeg = INT64_MAX;
        kend = INT64_MIN;
        Pmax = 0;
#pragma unroll
        for (int i = 0; i < kQueriesPerBlock; ++i) {
            kbeg = wlo[i] < kbeg ? wlo[i] : kbeg;
            kend = whi[i] > kend ? whi[i] : kend;
            const int64_t Pi = whi[i] > wlo[i] ? whi[i] - wlo[i] : 0;
            Pmax = Pi > Pmax ? Pi : Pmax;
        }
        if (kend <= kbeg) kbeg = kend = 0;
    } else {
        pos = p.q_pos0 + t;
        Pq = active ? visible_keys(pos, p.T, p.m, p.causal) : 0;
        int64_t last = grp * kQueriesPerBlock + kQueriesPerBlock - 1;
        if (last > p.nrows - 1) last = p.nrows - 1;
        const int64_t Pblk = visible_keys(p.q_pos0 + p.row0 + last, p.T, p.m, p.causal);
        kbeg = FEW ? (int64_t)sp * p.split_keys : 0;
        kend = FEW && kbeg + p.split_keys < Pblk ? kbeg + p.split_keys : Pblk;
        Pmax = Pblk;
    }
    // The end of an output row after its `body` selected entries: the tail
    // positions of the incomplete pool (clipped to the row for packed
    // documents, whose pools the caller forms), then -1; and valid_len.
    auto end_row = [&](int body, float *srow) {
        int tl = (p.expand && p.tail && p.causal) ? (int)(pos + 1 - Pq * p.m) : 0;
        if (VARLEN) tl = tl < 0 ? 0 : (tl > p.W - body ? p.W - body : tl);  // keys missing: clip
        int32_t *orow = p.idx + t * (int64_t)p.W;
        for (int s = body + lane; s < p.W; s += 64) {
            const bool in_tail = s < body + tl;
            orow[s] = in_tail ? (int32_t)(tok0 + Pq * p.m + (s - body)) : -1;
            if (srow) srow[s] = 0.f;
        }
        if (lane == 0) p.valid_len[t] = body + tl;
    };
    // No row of the block sees more keys than it selects and no score is
    // asked for: every visible key is selected whatever its score, so the
    // block loads nothing, scores nothing and writes its rows' visible keys
    // in key order (block-uniform, after the last barrier of such a block).
    if (!FEW && !p.sel_score && Pmax <= p.ksel) {
        if (active) {
            const int mexp = p.expand ? p.m : 1;
            const int64_t obase = VARLEN && p.expand ? tok0 - klo * p.m : 0;
            int32_t *orow = p.idx + t * (int64_t)p.W;
            for (int64_t j = lane; j < Pq; j += 64)
                for (int x = 0; x < mexp; ++x)
                    orow[j * mexp + x] = (int32_t)(obase + (klo + j) * mexp + x);
            end_row((int)Pq * mexp, nullptr);
        }
        return;
    }
    const int64_t khi = klo + Pq;
    const int ntiles = kend > kbeg ? (int)((kend - kbeg + kKeysPerTile - 1) / kKeysPerTile) : 0;

    uint32_t *hist = hist_all[wave];
    if (!FEW) hist_clear(hist, lane);

    // q fragments and folded head weights of this wave's query; every load
    // is issued from a clamped, valid address and masked afterwards, so the
    // loads are in flight together rather than one branch and wait each
    A qa[NB][KS];
    float wv[NB][16];
    const char *qbytes = static_cast<const char *>(p.q);
    const int64_t tq = active ? t : p.row0;
    // screening: A rows follow the certificate's head order (kept heads in
    // block 0), weights come from the certificate (w * q_scale, permuted)
    const int64_t crow = active ? qrow : 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int head = SCREEN ? p.cert_perm[crow * 64 + 32 * b + l32] : 32 * b + l32;
        const bool okq = active && head >= 0 && head < p.H;
        O::load_a(qbytes + ((tq * p.H + (okq ? head : 0)) * (int64_t)D) * ES, hh, qa[b]);
        if (!okq) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qa[b][ks] = O::zero();
        }
        if constexpr (SCREEN) {
            // the certificate's aggregate row: its values are operand values
            // already (bf16-representable, or fp32), in load_a's slot order
            if (active && head == kAggSlot) {
                const float *ag = p.cert_agg + crow * D + hh * (D / 2);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if constexpr (DT == 0) {
                        qa[b][ks] = ag[ks];
                    } else {
                        A v;
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = (__bf16)ag[ks * 8 + e];
                        qa[b][ks] = v;
                    }
                }
            }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int h2 = 32 * b + 8 * (v >> 2) + 4 * hh + (v & 3);
            const bool ok = active && h2 < p.H;
            const int hc = ok ? h2 : 0;
            if constexpr (SCREEN) {
                wv[b][v] = active ? p.cert_w[crow * 64 + h2] : 0.f;
            } else {
                float wt = p.w[tq * p.w_stride + hc];
                if (kScaled) wt *= p.q_scale[tq * p.H + hc];
                wv[b][v] = ok ? wt : 0.f;
            }
        }
    }
    // screening: folded bound weights of the kept heads and the key-norm
    // coefficient (residual allowance plus rounding margin)
    float wtb[16];
    float emu = 0.f;
    if constexpr (SCREEN) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
            wtb[v] = active ? p.cert_wt[crow * 32 + 8 * (v >> 2) + 4 * hh + (v & 3)] : 0.f;
        emu = active ? p.cert_e[crow] : 0.f;
    }

    uint2 *buf = p.ws + (active ? qrow : 0) * (int64_t)p.cap;
    // few-query mode: the row's estimate and the scores of the current
    // candidate batch (two tiles)
    const uint32_t west = FEW && active ? p.est[qrow] : 0u;
    float bsc[2];
    bsc[0] = bsc[1] = 0.f;
    int cnt = 0;
    uint32_t tau = 0;        // pass iff code >= tau
    float tau_f = -__builtin_inff();  // the same test on the float score
    bool tracking = false;   // cnt has reached ksel: tb / above are maintained
    int tb = 0, above = 0;   // boundary bin of the running histogram, count above it
    const int approx_limit = (p.cap + p.ksel) / 2;  // <= cap - kSelGroup: cap >= ksel + 4 groups

    const char *kbytes = static_cast<const char *>(p.k);
    uint4 stage[CPT];
    float ksc = 0.f, kn = 0.f;
    // bf16: a tile wholly below T is loaded unchecked off a uniform base with
    // per-thread offsets fixed for the launch (measured no better for fp8)
    constexpr bool kFastLoad = DT == 1;
    uint32_t goff[kFastLoad ? CPT : 1];
#pragma unroll
    for (int c = 0; c < (kFastLoad ? CPT : 1); ++c) {
        const int id = threadIdx.x + c * kThreads;
        goff[c] = (uint32_t)((id / GCH) * ROWB + (id % GCH) * 16);
    }
    auto load_tile = [&](int it) {
        const int64_t j0 = kbeg + (int64_t)it * kKeysPerTile;
        if (kFastLoad && j0 + kKeysPerTile <= p.T) {
            const char *tb = kbytes + j0 * ROWB;
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const int id = threadIdx.x + c * kThreads;
                if (id < GTILE_CH) stage[c] = *reinterpret_cast<const uint4 *>(tb + goff[c]);
            }
        } else {
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const int id = threadIdx.x + c * kThreads;
                stage[c] = make_uint4(0, 0, 0, 0);
                if (id < GTILE_CH) {
                    const int64_t key = j0 + id / GCH;
                    if (key < p.T)
                        stage[c] = reinterpret_cast<const uint4 *>(kbytes + key * ROWB)[id % GCH];
                }
            }
        }
        if (kScaled && threadIdx.x < kKeysPerTile) {
            const int64_t key = j0 + threadIdx.x;
            ksc = key < p.T ? p.k_scale[key] : 0.f;
        }
        if (SCREEN && threadIdx.x < kKeysPerTile) {
            const int64_t key = j0 + threadIdx.x;
            kn = key < p.T ? p.knorm[key] : 0.f;
        }
    };
    auto store_tile = [&](int slot) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int id = threadIdx.x + c * kThreads;
            if (id < GTILE_CH) {
                const int r = id / GCH;
                O::store_chunk(ktile[slot], r, id % GCH, stage[c], r & SWZ);
            }
        }
        if (kScaled && threadIdx.x < kKeysPerTile) kscale_tile[slot][threadIdx.x] = ksc;
        if (SCREEN && threadIdx.x < kKeysPerTile) knorm_tile[slot][threadIdx.x] = kn;
    };

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    // B operand reads: the XOR swizzle of a lane's rows (32 cb + l32) is
    // l32 & SWZ for every column block, so the byte offsets of its KS chunks
    // are fixed for the whole launch; a column block adds a constant.
    constexpr bool kBOff = DT != 0 && SWZ < 32;
    constexpr int NOFF = kBOff ? KS * CPK : 1;
    uint32_t boff[NOFF];
#pragma unroll
    for (int c = 0; c < NOFF; ++c)
        boff[c] = (uint32_t)((l32 * NCH + ((hh * KS * CPK + c) ^ (l32 & SWZ))) * 16);
    // B operand ks of column block cb from the staged tile at those offsets
    auto lds_b = [&](const char *tbytes, int cb, int ks) __attribute__((always_inline)) {
        uint4 ch[CPK > 0 ? CPK : 1];
#pragma unroll
        for (int c = 0; c < CPK; ++c)
            ch[c] = *reinterpret_cast<const uint4 *>(tbytes + cb * 32 * NCH * 16 +
                                                     boff[ks * CPK + c]);
        return O::from_chunks(ch);
    };

    // Selection of one tile's scores (NG groups of 64 keys, one key per lane).
    constexpr int NCB = kKeysPerTile / 32;  // 32-key column blocks per tile
    constexpr int NG = NCB / 2;             // 64-key selection groups per tile
    // One selection step: each lane offers one (score, key), ok = the key
    // is visible to this row; keys arrive in ascending order across calls.
    auto consider = [&](float sc, int64_t key, bool ok) __attribute__((always_inline)) {
        const uint32_t bits = __float_as_uint(sc);
        const bool pass = sc >= tau_f && ok;
        const uint64_t mask = __ballot(pass);
        if (mask) {
            const uint32_t u = ord_code(bits);
            if (pass) {
                buf[cnt + lane_rank(mask)] = make_uint2(bits, (uint32_t)key);
                hist_add(hist, u >> kShift1);
            }
            cnt += __popcll(mask);
            if (tracking) {
                // keep tau near the edge of the bin holding the Ksel-th best;
                // the boundary may lag by up to one group of entries
                above += __popcll(__ballot(pass && (int)(u >> kShift1) > tb));
                if (above >= p.ksel + kSelGroup) {
                    advance_boundary(hist, p.ksel, lane, tb, above);
                    const uint32_t edge = (uint32_t)tb << kShift1;
                    tau = edge > tau ? edge : tau;
                    tau_f = code_floor_value(tau);
                }
            } else if (cnt >= p.ksel) {
                tracking = true;
                int hb;
                find_boundary(hist, kBins1, p.ksel, lane, tb, above, hb);
                const uint32_t edge = (uint32_t)tb << kShift1;
                tau = edge > tau ? edge : tau;
                tau_f = code_floor_value(tau);
            }
            if (cnt > p.cap - kSelGroup) {  // overflow fallback
                wave_sync_mem();
                const Cut cut = choose_cut(buf, cnt, p.ksel, hist, true, approx_limit, lane);
                compact(buf, cnt, cut, hist, lane);
                tau = cut.tc + 1;
                tau_f = code_floor_value(tau);
                int hb;
                find_boundary(hist, kBins1, p.ksel, lane, tb, above, hb);
            }
        }
    };
    auto select_tile = [&](const float (&sg)[NG], int64_t j0) {
        if constexpr (FEW) {
            // the first tile of a batch waits for the second; the batch is
            // appended after its last tile this row reaches in this range
            static_assert(2 * NG * kSelGroup == kFewBatch, "two tiles per candidate batch");
            const bool second = (j0 / kKeysPerTile) & 1;
            const bool last = second || j0 + kKeysPerTile >= Pq || j0 + kKeysPerTile >= kend;
            if (!last) {
                bsc[0] = sg[0];
                bsc[1] = sg[1];
                return;
            }
            const int64_t b = j0 / kFewBatch;
            float sc[2 * NG];
            sc[0] = second ? bsc[0] : sg[0];
            sc[1] = second ? bsc[1] : sg[1];
            sc[2] = second ? sg[0] : 0.f;
            sc[3] = second ? sg[1] : 0.f;
            const int64_t kv = b * kFewBatch + (second ? 2 : 1) * kKeysPerTile;
            const int sub = (int)(b % kFewSub);
            fq_append<2 * NG>(sc, b * kFewBatch, Pq < kv ? Pq : kv, west,
                              p.fq_cnt + qrow * kFewSub + sub, buf + sub * kFewSubCap,
                              p.fq_dir + qrow * p.nbatch + b, lane, kFewSubCap);
            return;
        }
        const bool full = j0 >= klo && j0 + kKeysPerTile <= khi;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int64_t key = j0 + g * kSelGroup + lane;
            consider(sg[g], key, full || (key >= klo && key < khi));
        }
    };

    // Screened tile (DoSA summary, "Method steps": certificate screening and
    // survivor rescoring).  Block 0 holds the certificate's kept heads: their
    // MFMAs and signed-ReLU sum run for every key, and the same ReLU values
    // give the bound U = sum_kept w~ ReLU(x) + emu * ||k|| (times k_scale).
    // A key with U < tau cannot enter the selection, since its exact score
    // is at most U and tau never exceeds the final Ksel-th score; the others
    // are gathered 32 per MFMA column block, get block 1's heads (B read
    // from the staged tile at the survivor's row), and continue the exact
    // sum from their block-0 partial in the same order as an unscreened
    // tile, so a survivor's score does not depend on the screen.
    // screening statistics of this wave's row: keys tested against the
    // bound, keys that passed it
    uint32_t scr_tested = 0, scr_passed = 0;
    auto screen_tile = [&](int cur, int64_t j0) __attribute__((always_inline)) {
        constexpr int EPK = (16 + KS - 1) / KS;
        float part[NCB], ub[NCB];
        A bfr[KS];
        const char *tbytes = reinterpret_cast<const char *>(ktile[cur]);
        if constexpr (kBOff) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                bfr[ks] = lds_b(tbytes, 0, ks);
        } else {
            O::load_b(ktile[cur], l32, hh, l32 & SWZ, bfr);
        }
        f32x16 accp;
#pragma unroll
        for (int s = 0; s <= NCB; ++s) {  // MFMAs of column block s, epilogue of s - 1
            const bool loads = s + 1 < NCB;
            f32x16 acc;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] = 0.f;
            float e = 0.f, u = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (s < NCB) acc = O::mma(qa[0][ks], bfr[ks], acc);
                if (loads) {
                    if constexpr (kBOff) {
                        bfr[ks] = lds_b(tbytes, s + 1, ks);
                    } else {
                        const int r = (s + 1) * 32 + l32;
                        O::load_b_one(ktile[cur], r, hh, r & SWZ, ks, bfr[ks]);
                    }
                }
                if (s > 0) {
#pragma unroll
                    for (int x = 0; x < EPK; ++x) {
                        const int v = ks * EPK + x;
                        if (v < 16) {
                            const float r = fmaxf(accp[v], 0.f);
                            e = fmaf(wv[0][v], r, e);
                            u = fmaf(wtb[v], r, u);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (s > 0) {
                part[s - 1] = e;
                ub[s - 1] = u;
            }
            if (s < NCB) accp = acc;
        }
        float *p0 = p0_all[wave];
        uint16_t *sl = sl_all[wave];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) p0[hh * kKeysPerTile + cb * 32 + l32] = part[cb];
        const bool full = j0 >= klo && j0 + kKeysPerTile <= khi;
        int ns = 0;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ub[2 * g]),
                                                             __float_as_uint(ub[2 * g + 1]),
                                                             false, false);
            const int kl = g * kSelGroup + lane;
            float U = __uint_as_float(sw[0]) + __uint_as_float(sw[1]) + emu * knorm_tile[cur][kl];
            if (kScaled) U *= kscale_tile[cur][kl];
            const int64_t key = j0 + kl;
            const bool vis = full || (key >= klo && key < khi);
            const bool surv = vis && U >= tau_f;
            const uint64_t m = __ballot(surv);
            scr_tested += __popcll(__ballot(vis));
            scr_passed += __popcll(m);
            if (surv) sl[ns + lane_rank(m)] = (uint16_t)kl;
            ns += __popcll(m);
        }
        wave_sync_mem();
        // 64 survivors per round: two gathered column blocks (survivors
        // sb + 32c + l32), the MFMAs of the second issued with the epilogue
        // of the first, then the two lane halves added as for a plain tile
        int sb = 0;
        for (; sb + 32 < ns; sb += 2 * 32) {
            int kl[2];
            float pc[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int i = sb + 32 * c + l32;
                kl[c] = sl[i < ns ? i : sb];
                pc[c] = p0[hh * kKeysPerTile + kl[c]];
            }
            O::load_b(ktile[cur], kl[0], hh, kl[0] & SWZ, bfr);
#pragma unroll
            for (int s = 0; s <= 2; ++s) {  // MFMAs of gathered block s, epilogue of s - 1
                f32x16 acc;
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[v] = 0.f;
                float e = s > 0 ? pc[s - 1] : 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (s < 2) acc = O::mma(qa[1][ks], bfr[ks], acc);
                    if (s == 0) O::load_b_one(ktile[cur], kl[1], hh, kl[1] & SWZ, ks, bfr[ks]);
                    if (s > 0) {
#pragma unroll
                        for (int x = 0; x < EPK; ++x) {
                            const int v = ks * EPK + x;
                            if (v < 16) e = fmaf(wv[1][v], fmaxf(accp[v], 0.f), e);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (s > 0) pc[s - 1] = e;
                if (s < 2) accp = acc;
            }
            // lane L < 32: survivor sb + L from block 0; lane L >= 32: survivor
            // sb + L from block 1 -- the same lane's kl[hh]
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pc[0]),
                                                             __float_as_uint(pc[1]), false, false);
            const int klane = hh ? kl[1] : kl[0];
            float sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            if (kScaled) sc *= kscale_tile[cur][klane];
            consider(sc, j0 + klane, sb + lane < ns);
        }
        if (sb < ns) {  // at most 32 survivors left: one gathered block
            const int i = sb + l32;
            const int kl = sl[i < ns ? i : sb];
            O::load_b(ktile[cur], kl, hh, kl & SWZ, bfr);
            f32x16 acc;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = O::mma(qa[1][ks], bfr[ks], acc);
            float e = p0[hh * kKeysPerTile + kl];
#pragma unroll
            for (int v = 0; v < 16; ++v) e = fmaf(wv[1][v], fmaxf(acc[v], 0.f), e);
            // both lane halves of survivor sb + l32 meet in lanes l32 < 32
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(e),
                                                             __float_as_uint(e), false, false);
            float sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            if (kScaled) sc *= kscale_tile[cur][kl];
            consider(sc, j0 + kl, lane < 32 && i < ns);
        }
        wave_sync_mem();  // the next tile's survivor list reuses sl and p0
    };

    // The two waves sharing a SIMD (w and w + 4) run their selection at
    // opposite ends of a tile: waves 0-3 right after their MFMA/epilogue work,
    // waves 4-7 one tile later, before their MFMAs -- so one wave's branchy
    // selection code always has the other wave's MFMAs to overlap with.
    const bool lagged = !FEW && !SCREEN && wave >= kQueriesPerBlock / 2;
    float pend[NG];
    int64_t pend_j0 = -1;

    for (int it = 0; it < ntiles; ++it) {
        const int cur = it & 1;
        const int64_t j0 = kbeg + (int64_t)it * kKeysPerTile;
        if (it + 1 < ntiles) load_tile(it + 1);

        if (lagged && pend_j0 >= 0) {
            select_tile(pend, pend_j0);
            pend_j0 = -1;
        }
        if (SCREEN && active && j0 < khi && j0 + kKeysPerTile > klo) {
            screen_tile(cur, j0);
        } else if (active && j0 < khi && j0 + kKeysPerTile > klo) {
            // Software pipeline over steps (cb, b): the MFMAs of step s run
            // while the signed-ReLU epilogue of step s-1 is issued between
            // them; B of the next column block is fetched during the last
            // step that reads the current one.
            constexpr int NS = NCB * NB;
            float part[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) part[cb] = 0.f;
            // The wave in its MFMA phase issues first on its SIMD; the other
            // wave's selection fills the issue slots its MFMAs leave.
            __builtin_amdgcn_s_setprio(1);
            A bfr[KS];
            const char *tbytes = reinterpret_cast<const char *>(ktile[cur]);
            if constexpr (kBOff) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    bfr[ks] = lds_b(tbytes, 0, ks);
            } else {
                O::load_b(ktile[cur], l32, hh, l32 & SWZ, bfr);
            }
            f32x16 accp;
            constexpr int EPK = (16 + KS - 1) / KS;  // epilogue elements per MFMA slot
#pragma unroll
            for (int s = 0; s <= NS; ++s) {
                const int cb = s / NB, b = s % NB;
                const int pcb = (s - 1) / NB, pb = (s - 1) % NB;
                const bool loads = s < NS && b == NB - 1 && cb + 1 < NCB;
                f32x16 acc;
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[v] = 0.f;
                float e = s > 0 ? part[pcb] : 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (s < NS) acc = O::mma(qa[b][ks], bfr[ks], acc);
                    if (loads) {
                        if constexpr (kBOff) {
                            bfr[ks] = lds_b(tbytes, cb + 1, ks);
                        } else {
                            const int r = (cb + 1) * 32 + l32;
                            O::load_b_one(ktile[cur], r, hh, r & SWZ, ks, bfr[ks]);
                        }
                    }
                    if (s > 0) {
#pragma unroll
                        for (int x = 0; x < EPK; ++x) {
                            const int v = ks * EPK + x;
                            if (v < 16) e = fmaf(wv[pb][v], fmaxf(accp[v], 0.f), e);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (s > 0) part[pcb] = e;
                if (s < NS) accp = acc;
            }
            __builtin_amdgcn_s_setprio(0);
            float sg[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                // lanes < 32 finish keys 0..31 of this 64-key group, lanes >= 32
                // keys 32..63: swap the upper half of part[2g] with the lower
                // half of part[2g+1] and add
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[2 * g]),
                                                                 __float_as_uint(part[2 * g + 1]),
                                                                 false, false);
                sg[g] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                if (kScaled) sg[g] *= kscale_tile[cur][g * kSelGroup + lane];
            }
            if (lagged) {
#pragma unroll
                for (int g = 0; g < NG; ++g) pend[g] = sg[g];
                pend_j0 = j0;
            } else {
                select_tile(sg, j0);
            }
        }
        if (it + 1 < ntiles) store_tile(cur ^ 1);
        __syncthreads();
    }
    if (pend_j0 >= 0) select_tile(pend, pend_j0);
    if (SCREEN && p.scr_stats && lane == 0 && scr_tested) {
        atomicAdd(p.scr_stats, (unsigned long long)scr_tested);
        atomicAdd(p.scr_stats + 1, (unsigned long long)scr_passed);
    }

    if (!active || FEW) return;

    // ---- exact final selection, written straight into the output row ----
    // The K tiles are idle after the last barrier: each wave borrows a slice
    // of them to gather the codes of its boundary histogram bin.
    constexpr int kGatherCap = (int)(sizeof(ktile) / kQueriesPerBlock / sizeof(uint32_t));
    uint32_t *gather = reinterpret_cast<uint32_t *>(&ktile[0][0]) + wave * kGatherCap;
    wave_sync_mem();
    Cut cut;
    cut.tc = 0;
    cut.exact = 0;
    cut.need_eq = 0;
    if (cnt > p.ksel) cut = final_cut(buf, cnt, p.ksel, hist, gather, kGatherCap, lane);
    wave_sync_mem();

    const int mexp = p.expand ? p.m : 1;
    const int64_t obase = VARLEN && p.expand ? tok0 - klo * p.m : 0;  // key -> output index
    int32_t *orow = p.idx + t * (int64_t)p.W;
    float *srow = p.sel_score ? p.sel_score + t * (int64_t)p.W : nullptr;
    int wcnt = 0, eqseen = 0;
    for_each_entry(buf, cnt, lane, [&](bool valid, uint2 v) {
        const uint32_t u = ord_code(v.x);
        bool keep;
        if (cut.exact) {
            const bool eq = valid && u == cut.tc;
            const uint64_t em = __ballot(eq);
            keep = valid && (u > cut.tc || (eq && eqseen + lane_rank(em) < cut.need_eq));
            eqseen += __popcll(em);
        } else {
            keep = valid && u >= cut.tc;
        }
        const uint64_t km = __ballot(keep);
        if (keep) {
            const int o = (wcnt + lane_rank(km)) * mexp;
            for (int x = 0; x < mexp; ++x) {
                orow[o + x] = (int32_t)(obase + (int64_t)v.y * mexp + x);
                if (srow) srow[o + x] = __uint_as_float(v.x);
            }
        }
        wcnt += __popcll(km);
    });
    end_row(wcnt * mexp, srow);
}

template <int DT, int NB, int D, bool FEW, bool VARLEN, bool SCREEN>
hipError_t launch_one(const ScoreSelectParams &p, hipStream_t stream)
{
    const int64_t blocks = (p.nrows + kQueriesPerBlock - 1) / kQueriesPerBlock * p.nsplit;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((score_select_kernel<DT, NB, D, FEW, VARLEN, SCREEN>),
                       dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int DT, int NB, int D>
hipError_t launch_mode(bool few, bool varlen, bool screen, const ScoreSelectParams &p,
                       hipStream_t stream)
{
    if (varlen) return launch_one<DT, NB, D, false, true, false>(p, stream);
    if (few) return launch_one<DT, NB, D, true, false, false>(p, stream);
    if constexpr (NB == 2 && DT != 3) {
        if (screen) return launch_one<DT, NB, D, false, false, true>(p, stream);
    }
    return launch_one<DT, NB, D, false, false, false>(p, stream);
}

}  // namespace

hipError_t launch_score_select(int dtype, int nb, int d, bool few, bool varlen, bool screen,
                               const ScoreSelectParams &p, hipStream_t stream, bool *supported)
{
    *supported = true;
    if (p.nsplit < 1 || p.split_keys < kKeysPerTile || p.split_keys % kKeysPerTile ||
        (varlen && (few || p.nsplit != 1)) || (screen && (few || varlen || nb != 2))) {
        *supported = false;
        return hipSuccess;
    }
#define DSAI_CASE(DT, NB, D) \
    if (dtype == DT && nb == NB && d == D) \
        return launch_mode<DT, NB, D>(few, varlen, screen, p, stream);
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
