"""Seeded sweep of small integer-valued problems over every mode and path,
compared with the oracle bit for bit.

Small integers in every dtype (fp32, bf16, and e4m3 codes with scales in
{1/2, 1, 2}) make every product and every sum exact in any order (at most
22 significant bits at d = 128, H = 64), so the top-k
under the tie rule (higher score, then lower index) is unique and the HIP
path must reproduce the oracle's rows exactly: indices, valid lengths and
selected scores.  Each case draws the shape (S, T, H, d, m, topk), the mode
(causal, expansion, tail, query offset, broadcast or per-row weights), the
path knobs (query chunk, few-query rows, screening) and whether selected
scores are asked for; the case id names its seed.  A second sweep packs
random documents (lengths, first positions, padding rows, fewer keys than
pools) and compares the varlen call with the oracle's per-document
composition, on the streaming and the few-query path, with and without a
bound on keys per document.
"""
import numpy as np
import pytest
import torch

from gpu_util import log, run
from oracle import check
from oracle import oracle as orc
from workloads import gen

pytestmark = pytest.mark.gpu
DEV = "cuda"
NCASES = 160


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = [torch.float32, torch.bfloat16, torch.float8_e4m3fn][seed % 3]
    d = int(rng.choice([32, 64] if dtype == torch.float32 else [32, 64, 128]))
    H = int(rng.choice([1, 3, 8, 32, 33, 48, 64]))
    m = int(rng.choice([1, 1, 2, 4, 8]))
    causal = bool(rng.random() < 0.8)
    expand = bool(m > 1 and rng.random() < 0.6)
    tail = bool(expand and causal and rng.random() < 0.7)
    S = int(rng.integers(1, 700))
    q_pos0 = int(rng.integers(0, 400)) if causal and rng.random() < 0.5 else 0
    T = int(rng.integers(1, 900))
    if tail:
        T = max(T, (q_pos0 + S) // m)
    ksel = int(rng.choice([1, 7, 64, 200, 1000]))
    topk = ksel * m if expand else ksel
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(-3, 4, (S, H, d), generator=g).float()
    k = torch.randint(-3, 4, (T, d), generator=g).float()
    wv = torch.tensor([-1.0, -0.5, 0.5, 1.0])
    w = wv[torch.randint(0, 4, (H,) if rng.random() < 0.5 else (S, H), generator=g)]
    qs = ks = None
    if dtype == torch.float8_e4m3fn:
        qs = 2.0 ** torch.randint(-1, 2, (S, H), generator=g).float()
        ks = 2.0 ** torch.randint(-1, 2, (T,), generator=g).float()
    q, k = q.to(dtype), k.to(dtype)
    inp = gen.custom(q=q, k=k, w=w, m=m, topk=topk, causal=causal, expand=expand, tail=tail,
                     q_scale=qs, k_scale=ks, q_pos0=q_pos0)
    knobs = dict(query_chunk=int(rng.choice([0, 0, 64, 257])),
                 few_query_rows=int(rng.choice([0, -1, 700])),
                 screen=bool(rng.random() < 0.3),
                 with_scores=bool(rng.random() < 0.6))
    return inp, knobs


@pytest.mark.parametrize("seed", range(NCASES))
def test_integer_sweep_matches_oracle_exactly(seed):
    inp, knobs = _case(seed)
    log(f"  seed {seed}: {inp.dtype} S={inp.S} T={inp.T} H={inp.H} d={inp.d} m={inp.m} "
        f"topk={inp.topk} causal={inp.causal} expand={inp.expand} tail={inp.tail} "
        f"q_pos0={inp.q_pos0} {knobs}")
    inp = inp.to(DEV)
    out = run(inp, **knobs)
    idx, vl = out[0], out[1]
    sc = out[2] if knobs["with_scores"] else None
    rows = np.arange(inp.S)
    ref = orc.select_rows(inp, rows)
    rep = check.compare(inp, rows, idx.cpu().numpy(), vl.cpu().numpy(),
                        None if sc is None else sc.cpu().numpy(), exact=True, ref=ref)
    assert rep["ok"], rep["failures"][:3]
    if sc is not None:
        # exact inputs: each selected key's reported score is the oracle's
        # score exactly (repeated over its m positions), tail and padding 0;
        # the oracle lists its selection by rank, the output by key
        got, vlh = sc.cpu().numpy(), vl.cpu().numpy()
        mexp = inp.m if inp.expand else 1
        for r in range(inp.S):
            n = int(ref["n_sel"][r])
            order = np.argsort(ref["key_idx"][r][:n], kind="stable")
            want = np.repeat(ref["key_score"][r][:n][order], mexp)
            assert np.array_equal(got[r, :n * mexp], want.astype(np.float32)), r
            assert not got[r, n * mexp:].any(), r
            assert int(vlh[r]) >= n * mexp


def _varlen_case(seed):
    rng = np.random.default_rng(5000 + seed)
    dtype = [torch.float32, torch.bfloat16, torch.float8_e4m3fn][seed % 3]
    d = int(rng.choice([32, 64] if dtype == torch.float32 else [32, 64, 128]))
    H = int(rng.choice([1, 4, 32, 48, 64]))
    m = int(rng.choice([1, 2, 4]))
    causal = bool(rng.random() < 0.85)
    expand = bool(m > 1 and rng.random() < 0.6)
    tail = bool(expand and causal and rng.random() < 0.7)
    ndoc = int(rng.integers(1, 12))
    lens = rng.choice([1, 2, 3, 5, 8, 17, 64, 100, 300, 700], size=ndoc).astype(np.int64)
    pos0 = rng.integers(0, 50, size=ndoc) if causal and rng.random() < 0.5 else \
        np.zeros(ndoc, np.int64)
    if causal:
        nkeys = (pos0 + lens) // m                          # every complete pool
        if not tail and rng.random() < 0.3:                 # or fewer keys than pools
            nkeys = nkeys - rng.integers(0, nkeys // 2 + 1)
    else:
        nkeys = rng.integers(1, 400, size=ndoc)
    nkeys[int(rng.integers(0, ndoc))] += 1                  # at least one key
    S = int(lens.sum()) + int(rng.integers(0, 4))           # padding rows
    T = int(nkeys.sum())
    cu_q = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(nkeys)]).astype(np.int32)
    cu_tok = np.concatenate([[0], np.cumsum(pos0 + lens)])[:-1].astype(np.int32)
    ksel = int(rng.choice([1, 7, 64, 200]))
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(-3, 4, (S, H, d), generator=g).float()
    k = torch.randint(-3, 4, (T, d), generator=g).float()
    wv = torch.tensor([-1.0, -0.5, 0.5, 1.0])
    w = wv[torch.randint(0, 4, (H,) if rng.random() < 0.5 else (S, H), generator=g)]
    qs = ks = None
    if dtype == torch.float8_e4m3fn:
        qs = 2.0 ** torch.randint(-1, 2, (S, H), generator=g).float()
        ks = 2.0 ** torch.randint(-1, 2, (T,), generator=g).float()
    inp = gen.custom(q=q.to(dtype), k=k.to(dtype), w=w, m=m, topk=ksel * m if expand else ksel,
                     causal=causal, expand=expand, tail=tail, q_scale=qs, k_scale=ks)
    most = int(nkeys.max())
    knobs = dict(few_query_rows=int(rng.choice([0, -1, 10000])),
                 max_doc_keys=int(rng.choice([0, most, most + 17])),
                 with_scores=bool(rng.random() < 0.5))
    return inp, (cu_q, cu_k, pos0.astype(np.int64), cu_tok), knobs


@pytest.mark.parametrize("seed", range(NCASES // 2))
def test_varlen_integer_sweep_matches_oracle_exactly(seed):
    import dsa_indexer_score_amd as dsai
    inp, (cu_q, cu_k, pos0, cu_tok), knobs = _varlen_case(seed)
    log(f"  seed {seed}: {inp.dtype} S={inp.S} T={inp.T} H={inp.H} d={inp.d} m={inp.m} "
        f"topk={inp.topk} causal={inp.causal} expand={inp.expand} tail={inp.tail} "
        f"docs={len(cu_q) - 1} {knobs}")
    inp = inp.to(DEV)
    t = lambda a, dt: torch.as_tensor(a, dtype=dt, device=DEV)
    ix = dsai.Indexer(inp.q.dtype, expand=inp.expand, tail=inp.tail,
                      few_query_rows=knobs["few_query_rows"], device=DEV)
    out = ix.score_topk_varlen(inp.q, inp.w, inp.k, t(cu_q, torch.int32), t(cu_k, torch.int32),
                               m=inp.m, topk=inp.topk, causal=inp.causal,
                               pos0=t(pos0, torch.int64),
                               cu_tok=t(cu_tok, torch.int32) if inp.expand else None,
                               q_scale=inp.q_scale, k_scale=inp.k_scale,
                               max_doc_keys=knobs["max_doc_keys"],
                               with_scores=knobs["with_scores"])
    torch.cuda.synchronize()
    want = orc.select_rows_varlen(inp, cu_q, cu_k, pos0=pos0, cu_tok=cu_tok)
    assert np.array_equal(out[1].cpu().numpy(), want["valid_len"])
    assert np.array_equal(out[0].cpu().numpy(), want["idx"])
