"""Packed documents (varlen) on the GPU against the oracle.

GLM-5.3-Flash Module 06 "DSA & KPool", section 3 and "Ship it": the watch
lengths repeated inside packed multi-document batches, with padding, and no
cross-document leakage.  Integer-valued problems are compared bit for bit
with the oracle's per-document composition; float problems per document
under the tolerance rule; one document through the varlen call equals the
plain call bit for bit.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from gpu_util import log
from oracle import check
from oracle import oracle as orc
from workloads import gen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _layout(rng, lens, m, pos0=None):
    ndoc = len(lens)
    pos0 = np.zeros(ndoc, np.int64) if pos0 is None else np.asarray(pos0, np.int64)
    nkeys = [(int(p) + int(n)) // m for p, n in zip(pos0, lens)]   # every complete pool
    cu_q = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(nkeys)]).astype(np.int32)
    cu_tok = np.concatenate([[0], np.cumsum(pos0 + np.asarray(lens))])[:-1].astype(np.int32)
    return cu_q, cu_k, pos0, cu_tok


def _run(inp, cu_q, cu_k, pos0, cu_tok, with_scores=True, few=0, max_doc_keys=0):
    import dsa_indexer_score_amd as dsai
    ix = dsai.Indexer(inp.q.dtype, expand=inp.expand, tail=inp.tail,
                      query_chunk=inp.query_chunk or 0, few_query_rows=few, device=DEV)
    t = lambda a, dt: torch.as_tensor(np.asarray(a), dtype=dt, device=DEV)
    out = ix.score_topk_varlen(
        inp.q, inp.w, inp.k, t(cu_q, torch.int32), t(cu_k, torch.int32), m=inp.m, topk=inp.topk,
        causal=inp.causal, pos0=t(pos0, torch.int64),
        cu_tok=t(cu_tok, torch.int32) if inp.expand else None, q_scale=inp.q_scale,
        k_scale=inp.k_scale, max_doc_keys=max_doc_keys, with_scores=with_scores)
    torch.cuda.synchronize()
    return out


WATCH = [3, 4, 5, 7, 8, 9]


@pytest.mark.parametrize("m,expand,seed", [(4, True, 0), (4, False, 1), (1, False, 2),
                                           (4, True, 3)])
def test_varlen_integer_batches_match_oracle_exactly(m, expand, seed):
    rng = np.random.default_rng(100 + seed)
    lens = list(rng.choice(WATCH + [1, 2, 16, 63, 64, 65, 300], size=40))
    pos0 = rng.integers(0, 40, size=len(lens)) if seed == 3 else None
    cu_q, cu_k, pos0, cu_tok = _layout(rng, lens, m, pos0)
    S, T = int(cu_q[-1]) + 5, int(cu_k[-1])              # 5 padding rows
    H, d = 4, 32
    q = torch.from_numpy(rng.integers(-3, 4, size=(S, H, d)).astype(np.float32))
    k = torch.from_numpy(rng.integers(-3, 4, size=(T, d)).astype(np.float32))
    w = torch.from_numpy(rng.choice([-1.0, -0.5, 0.5, 1.0], size=(S, H)).astype(np.float32))
    topk = 12 if expand else 7
    inp = gen.custom(q=q, k=k, w=w, m=m, topk=topk, expand=expand, tail=expand).to(DEV)
    idx, vl, sc = _run(inp, cu_q, cu_k, pos0, cu_tok)
    want = orc.select_rows_varlen(inp, cu_q, cu_k, pos0=pos0, cu_tok=cu_tok)
    assert np.array_equal(vl.cpu().numpy(), want["valid_len"])
    assert np.array_equal(idx.cpu().numpy(), want["idx"])
    assert (vl[-5:] == 0).all() and (idx[-5:] == -1).all()
    log(f"  m={m} expand={expand}: {len(lens)} documents, S={S}, T={T}")


def test_one_document_equals_the_plain_call():
    import dsa_indexer_score_amd as dsai
    for name, S in (("c4_csa_256k", 3000), ("c2_glm_pooled", 2000), ("c3_dsa_token", 1500)):
        m = gen.CONFIGS[name]["m"]
        T = (37 + S) // m                       # every complete pool of the context
        inp = replace(gen.generate(name, S=S, T=T, topk=256), q_pos0=37).to(DEV)
        ref = dsai.score_topk(inp.q, inp.w, inp.k, m=inp.m, topk=inp.topk, causal=True,
                              expand=inp.expand, tail=inp.tail, q_scale=inp.q_scale,
                              k_scale=inp.k_scale, q_pos0=inp.q_pos0, few_query_rows=-1,
                              with_scores=True)
        got = _run(inp, [0, S], [0, T], [inp.q_pos0], [0])
        for a, b in zip(ref, got):
            assert torch.equal(a, b), name


@pytest.mark.parametrize("name", ["c4_csa_256k", "c2_glm_pooled"])
def test_varlen_float_batch_per_document(name):
    """A packed bf16 batch: every document's rows, mapped back to local
    indices, pass the tolerance rule against the oracle on that document."""
    rng = np.random.default_rng(7)
    base = gen.generate(name, S=6000, topk=512)
    m = base.m
    lens = [5, 1000, 3, 2048, 7, 400, 2500]
    cu_q, cu_k, pos0, cu_tok = _layout(rng, lens, m)
    S, T = int(cu_q[-1]), int(cu_k[-1])
    inp = replace(base, S=S, T=T, q=base.q[:S].contiguous(), k=base.k[:T].contiguous(),
                  k_scale=None if base.k_scale is None else base.k_scale[:T].contiguous()).to(DEV)
    idx, vl, sc = _run(inp, cu_q, cu_k, pos0, cu_tok)
    idx, vl, sc = idx.cpu().numpy(), vl.cpu().numpy(), sc.cpu().numpy()
    for i in range(len(lens)):
        r0, r1, k0, k1 = int(cu_q[i]), int(cu_q[i + 1]), int(cu_k[i]), int(cu_k[i + 1])
        sub = replace(inp, S=r1 - r0, T=k1 - k0, q=inp.q[r0:r1], k=inp.k[k0:k1],
                      w=inp.w if inp.w.dim() == 1 else inp.w[r0:r1],
                      k_scale=None if inp.k_scale is None else inp.k_scale[k0:k1])
        loc = idx[r0:r1].astype(np.int64)
        base_off = int(cu_tok[i]) if inp.expand else k0
        loc[loc >= 0] -= base_off
        rep = check.compare(sub, np.arange(r1 - r0), loc.astype(np.int32), vl[r0:r1],
                            sc[r0:r1])
        assert rep["ok"], (i, rep["failures"][:3])


def _decode_batch(rng, lens, m, dtype, H=8, d=64, pad=3):
    """One query row per document, at the last position of each document's
    context (batched decode), plus padding rows."""
    lens = np.asarray(lens, np.int64)
    nkeys = lens // m                                     # complete pools only
    cu_k = np.concatenate([[0], np.cumsum(nkeys)]).astype(np.int32)
    ndoc = len(lens)
    cu_q = np.arange(ndoc + 1, dtype=np.int32)
    pos0 = lens - 1                                       # the row is the last token
    cu_tok = np.concatenate([[0], np.cumsum(lens)])[:-1].astype(np.int32)
    S, T = ndoc + pad, int(cu_k[-1])
    g = torch.Generator().manual_seed(int(rng.integers(1 << 30)))
    if dtype == torch.float32:
        q = torch.randint(-3, 4, (S, H, d), generator=g).float()
        k = torch.randint(-3, 4, (T, d), generator=g).float()
        w = torch.tensor(rng.choice([-1.0, -0.5, 0.5, 1.0], size=(S, H)), dtype=torch.float32)
        qs = ks = None
    else:
        q = torch.randn(S, H, d, generator=g) / d ** 0.5
        k = torch.randn(T, d, generator=g) / d ** 0.5
        w = torch.randn(S, H, generator=g)
        qs = ks = None
        if dtype == torch.float8_e4m3fn:
            qs = q.abs().amax(-1) / 448 + 1e-12
            ks = k.abs().amax(-1) / 448 + 1e-12
            q, k = q / qs[..., None], k / ks[:, None]
        q, k = q.to(dtype), k.to(dtype)
    return q, k, w, qs, ks, cu_q, cu_k, pos0, cu_tok


@pytest.mark.parametrize("m,expand", [(4, True), (4, False), (1, False)])
def test_batched_decode_few_query_path_is_exact(m, expand):
    """One row per document at the end of its context (lengths around the
    pool edges and long ones), padding rows: the few-query path equals the
    streaming path bit for bit and the oracle exactly (integer inputs)."""
    rng = np.random.default_rng(40 + m)
    lens = [3, 4, 5, 7, 8, 9, 64, 65, 900, 5000, 20000, 37]
    q, k, w, qs, ks, cu_q, cu_k, pos0, cu_tok = _decode_batch(rng, lens, m, torch.float32)
    topk = 48 if expand else 12
    inp = gen.custom(q=q, k=k, w=w, m=m, topk=topk, expand=expand, tail=expand).to(DEV)
    dense = _run(inp, cu_q, cu_k, pos0, cu_tok, few=64)
    stream = _run(inp, cu_q, cu_k, pos0, cu_tok, few=-1)
    for a, b in zip(dense, stream):
        assert torch.equal(a, b)
    want = orc.select_rows_varlen(inp, cu_q, cu_k, pos0=pos0, cu_tok=cu_tok)
    assert np.array_equal(dense[1].cpu().numpy(), want["valid_len"])
    assert np.array_equal(dense[0].cpu().numpy(), want["idx"])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float8_e4m3fn])
def test_batched_decode_float_matches_streaming(dtype):
    rng = np.random.default_rng(7)
    lens = [70000, 4096, 123457, 9, 30000, 65536]
    q, k, w, qs, ks, cu_q, cu_k, pos0, cu_tok = _decode_batch(rng, lens, 4, dtype, H=64, d=128)
    inp = gen.custom(q=q, k=k, w=w, m=4, topk=2048, expand=False, tail=False, q_scale=qs,
                     k_scale=ks).to(DEV)
    dense = _run(inp, cu_q, cu_k, pos0, cu_tok, few=64)
    stream = _run(inp, cu_q, cu_k, pos0, cu_tok, few=-1)
    for a, b in zip(dense, stream):
        assert torch.equal(a, b)
    log(f"  {dtype}: {len(lens)} decode rows over {int(cu_k[-1])} keys, valid_len "
        f"{dense[1].tolist()}")


def test_few_query_rows_of_several_documents():
    """Few rows, several per document, later-chunk positions and padding:
    few-query and streaming paths agree bit for bit."""
    rng = np.random.default_rng(8)
    lens = [5, 1, 20, 3]
    cu_q, cu_k, pos0, cu_tok = _layout(rng, lens, 4, pos0=[0, 33, 100, 7])
    S, T, H, d = int(cu_q[-1]) + 2, int(cu_k[-1]), 4, 32
    q = torch.from_numpy(rng.integers(-3, 4, size=(S, H, d)).astype(np.float32))
    k = torch.from_numpy(rng.integers(-3, 4, size=(T, d)).astype(np.float32))
    w = torch.from_numpy(rng.choice([-1.0, 1.0], size=(S, H)).astype(np.float32))
    inp = gen.custom(q=q, k=k, w=w, m=4, topk=16, expand=True, tail=True).to(DEV)
    dense = _run(inp, cu_q, cu_k, pos0, cu_tok, few=64)
    stream = _run(inp, cu_q, cu_k, pos0, cu_tok, few=-1)
    for a, b in zip(dense, stream):
        assert torch.equal(a, b)
    want = orc.select_rows_varlen(inp, cu_q, cu_k, pos0=pos0, cu_tok=cu_tok)
    assert np.array_equal(dense[0].cpu().numpy(), want["idx"])


def test_batched_decode_over_long_documents():
    """43 decode rows over 19.4M packed keys (a score array for them would
    take 3.3 GB; the few-query workspace holds about 30 MB: key samples,
    candidate lists and one directory entry per 256 keys); the result
    equals the streaming path bit for bit."""
    rng = np.random.default_rng(12)
    lens = rng.integers(1_000_000, 3_000_000, size=40)     # 19.4M complete pools
    q, k, w, qs, ks, cu_q, cu_k, pos0, cu_tok = _decode_batch(rng, lens, 4, torch.bfloat16,
                                                              H=4, d=32)
    inp = gen.custom(q=q, k=k, w=w, m=4, topk=512, expand=True, tail=True).to(DEV)
    import dsa_indexer_score_amd as dsai
    ix = dsai.Indexer(torch.bfloat16, expand=True, tail=True, few_query_rows=64, device=DEV)
    assert ix.workspace_bytes_varlen(inp.S, inp.T, 4, 32, 4, 512, len(lens)) < inp.S * inp.T
    dense = _run(inp, cu_q, cu_k, pos0, cu_tok, few=64)
    stream = _run(inp, cu_q, cu_k, pos0, cu_tok, few=-1)
    for a, b in zip(dense, stream):
        assert torch.equal(a, b)
    log(f"  {inp.S} rows over {inp.T} keys, valid_len {dense[1][:4].tolist()}...")


@pytest.mark.parametrize("m,expand", [(4, True), (1, False)])
def test_batched_decode_with_a_bound_on_document_keys(m, expand):
    """max_doc_keys sizes the dense rows by the longest document instead of
    all keys: 43 rows over about 20M packed keys then fit one pass; with the
    exact bound, a looser one and none the result is the same, bit for bit,
    and equals the streaming path."""
    rng = np.random.default_rng(13)
    lens = rng.integers(250_000, 750_000, size=40) * m     # about 20M complete pools
    q, k, w, qs, ks, cu_q, cu_k, pos0, cu_tok = _decode_batch(rng, lens, m, torch.bfloat16,
                                                              H=4, d=32)
    inp = gen.custom(q=q, k=k, w=w, m=m, topk=512, expand=expand, tail=expand).to(DEV)
    longest = int(np.diff(cu_k).max())
    import dsa_indexer_score_amd as dsai
    ix = dsai.Indexer(torch.bfloat16, expand=expand, tail=expand, few_query_rows=64, device=DEV)
    nb = ix.workspace_bytes_varlen(inp.S, inp.T, 4, 32, m, 512, len(lens), longest)
    assert nb < 13 * inp.S * longest                      # one pass of short rows
    ref = _run(inp, cu_q, cu_k, pos0, cu_tok, few=-1)
    for bound in (longest, longest + 12345, 0):
        got = _run(inp, cu_q, cu_k, pos0, cu_tok, few=64, max_doc_keys=bound)
        for a, b in zip(ref, got):
            assert torch.equal(a, b), bound
    log(f"  m={m}: {inp.S} rows, longest document {longest} keys of {inp.T}, "
        f"workspace {nb / 2 ** 20:.0f} MiB with the bound")


@pytest.mark.parametrize("m,expand", [(4, True), (1, False)])
def test_short_documents_need_no_scores(m, expand):
    """Documents whose rows see at most Ksel keys select every visible key:
    without sel_score their blocks write them unscored.  Mixed with longer
    documents and padding, the result equals the oracle exactly (integer
    inputs) and the scored call bit for bit."""
    rng = np.random.default_rng(70 + m)
    lens = list(rng.choice([1, 3, 4, 5, 9, 64, 100, 129, 130, 300], size=50)) + [700, 2000]
    cu_q, cu_k, pos0, cu_tok = _layout(rng, lens, m)
    S, T, H, d = int(cu_q[-1]) + 3, int(cu_k[-1]), 4, 32
    q = torch.from_numpy(rng.integers(-3, 4, size=(S, H, d)).astype(np.float32))
    k = torch.from_numpy(rng.integers(-3, 4, size=(T, d)).astype(np.float32))
    w = torch.from_numpy(rng.choice([-1.0, -0.5, 0.5, 1.0], size=(S, H)).astype(np.float32))
    topk = 32 * m if expand else 32                       # Ksel = 32 keys
    inp = gen.custom(q=q, k=k, w=w, m=m, topk=topk, expand=expand, tail=expand).to(DEV)
    plain = _run(inp, cu_q, cu_k, pos0, cu_tok, with_scores=False, few=-1)
    scored = _run(inp, cu_q, cu_k, pos0, cu_tok, with_scores=True, few=-1)
    assert torch.equal(plain[0], scored[0]) and torch.equal(plain[1], scored[1])
    want = orc.select_rows_varlen(inp, cu_q, cu_k, pos0=pos0, cu_tok=cu_tok)
    assert np.array_equal(plain[1].cpu().numpy(), want["valid_len"])
    assert np.array_equal(plain[0].cpu().numpy(), want["idx"])
