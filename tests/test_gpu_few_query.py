"""The few-query path (sampled threshold estimate, scoring with sparse
write-back of the keys that reach it, exact cut per row, repair of the rows
whose estimate fails by the streaming kernel) against the streaming path and
the oracle.

Both paths share the scoring arithmetic and implement the same exact
selection, so on the same inputs they must agree bit for bit (indices,
valid lengths and reported scores); decode-shaped rows -- a few queries at
the end of a long context, all keys visible -- are also compared with the
oracle on every row under the tolerance rule.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from gpu_util import log, run
from oracle import check
from workloads import gen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _decode(name, S, T, topk=None):
    """S query rows at the very end of a context whose keys are all complete."""
    inp = gen.generate(name, S=S, T=T, topk=topk)
    return replace(inp, q_pos0=T * inp.m - S).to(DEV)


def _both_paths(inp, **kw):
    dense = run(inp, few_query_rows=max(64, inp.S), **kw)
    stream = run(inp, few_query_rows=-1, **kw)
    return dense, stream


def _assert_identical(a, b):
    for x, y in zip(a, b):
        if x is None:
            assert y is None
            continue
        assert torch.equal(x, y)


CASES = [
    ("c4_csa_256k", 64, 65536, None),       # bf16 compressed keys, decode at 256K tokens
    ("c5_csa_1m", 7, 262144, None),         # fp8 compressed keys, decode at 1M tokens
    ("c3_dsa_token", 40, 131072, None),     # fp8 token keys
    ("c2_glm_pooled", 33, 8192, None),      # bf16 pooled keys, expansion + tail
    ("c1_tiny_int", 50, 1024, None),        # integer-valued fp32
    ("c4_csa_256k", 3, 1500, 4096),         # topk above every row's visible count
]


@pytest.mark.parametrize("name,S,T,topk", CASES)
def test_few_query_path_is_bit_identical_to_streaming(name, S, T, topk):
    inp = _decode(name, S, T, topk)
    dense, stream = _both_paths(inp)
    _assert_identical(dense, stream)
    log(f"  {name} S={S} T={T}: valid_len {dense[1].min().item()}..{dense[1].max().item()}")


DECODE_T = {"c4_csa_256k": 65536, "c5_csa_1m": 262144, "c3_dsa_token": 131072,
            "c2_glm_pooled": 8192, "c1_tiny_int": 1024}


@pytest.mark.parametrize("S", [1, 2])
@pytest.mark.parametrize("name", list(DECODE_T))
def test_one_and_two_rows_bit_identical_to_streaming(name, S):
    """One or two rows are scored by the register-resident row kernel; its
    scores, and so the selections, equal the streaming kernel's bit for bit."""
    inp = _decode(name, S, DECODE_T[name])
    _assert_identical(*_both_paths(inp))


@pytest.mark.parametrize("dtype,H,d", [(torch.float32, 17, 32), (torch.float32, 40, 64),
                                       (torch.bfloat16, 5, 32), (torch.bfloat16, 33, 64),
                                       (torch.float8_e4m3fn, 64, 32),
                                       (torch.float8_e4m3fn, 20, 64),
                                       (torch.float8_e4m3fn, 48, 128)])
def test_one_and_two_rows_every_operand_shape(dtype, H, d):
    """Every (dtype, head blocks, d) instance of the row kernel, with missing
    heads, a ragged key count and rows that do not see every key."""
    g = torch.Generator().manual_seed(H * 1000 + d)
    T = 3001
    for S in (1, 2):
        q = torch.randn(S, H, d, generator=g).to(dtype)
        k = torch.randn(T, d, generator=g).to(dtype)
        w = torch.randn(S, H, generator=g)
        fp8 = dtype == torch.float8_e4m3fn
        inp = gen.custom(q=q, k=k, w=w, topk=200, q_pos0=T - 40,
                         q_scale=torch.rand(S, H, generator=g) + 0.5 if fp8 else None,
                         k_scale=torch.rand(T, generator=g) + 0.5 if fp8 else None).to(DEV)
        _assert_identical(*_both_paths(inp))


def test_few_query_path_prefix_rows_and_non_causal():
    """Rows at the start of the context (few visible keys, empty rows) and a
    non-causal ragged problem take the same results through both paths."""
    inp = gen.generate("c4_csa_256k", S=40, T=3000).to(DEV)      # q_pos0 = 0: P_t tiny
    _assert_identical(*_both_paths(inp))
    inp = gen.generate("c2_glm_pooled", S=29, T=777).to(DEV)
    inp = replace(inp, causal=False, expand=False, tail=False)
    _assert_identical(*_both_paths(inp))


@pytest.mark.parametrize("name,S,T", [("c5_csa_1m", 1, 262144), ("c4_csa_256k", 2, 65536),
                                      ("c5_csa_1m", 3, 262144), ("c4_csa_256k", 8, 65536),
                                      ("c2_glm_pooled", 5, 8192)])
def test_decode_rows_match_oracle(name, S, T):
    inp = _decode(name, S, T)
    idx, vl, sc = run(inp, few_query_rows=64)
    rep = check.compare(inp, np.arange(S), idx.cpu().numpy(), vl.cpu().numpy(), sc.cpu().numpy())
    assert rep["ok"], rep["failures"]
    log(f"  {name} decode S={S}: max score rel err {rep['max_score_rel_err']:.2e}")


def test_few_query_ties_and_monotone_scores():
    """Every score equal (q = 0): the tie rule alone decides, across a run of
    equal codes far longer than the selection; ascending scores: the last
    keys win."""
    S, T, H, d = 5, 5000, 64, 64
    g = torch.Generator().manual_seed(3)
    k = torch.randn(T, d, generator=g).bfloat16()
    q = torch.zeros(S, H, d).bfloat16()
    w = torch.randn(H, generator=g)
    inp = replace(gen.custom(q=q, k=k, w=w, topk=100), q_pos0=T - S).to(DEV)
    idx, vl, sc = run(inp, few_query_rows=64)
    assert (vl.cpu() == 100).all()
    assert (idx.cpu() == torch.arange(100, dtype=torch.int32)).all()
    assert bool((sc == 0).all())
    q = torch.zeros(S, 1, 32)
    q[:, 0, 0] = 1.0
    k = torch.zeros(T, 32)
    k[:, 0] = torch.arange(T, dtype=torch.float32)
    inp = replace(gen.custom(q=q, k=k, w=torch.ones(1), topk=300), q_pos0=T - S).to(DEV)
    idx, vl, _ = run(inp, few_query_rows=64)
    for t in range(S):
        P = T - S + t + 1
        assert idx[t].cpu().tolist() == list(range(P - 300, P))


def test_few_query_empty_and_single_key():
    inp = gen.generate("c4_csa_256k", S=3, T=1).to(DEV)
    _assert_identical(*_both_paths(inp))
    idx, vl, _ = run(inp, few_query_rows=64)
    assert vl.tolist() == [0, 0, 0]               # positions 0..2 see no complete pool
    inp = replace(gen.generate("c4_csa_256k", S=4, T=1), q_pos0=3).to(DEV)
    idx, vl, _ = run(inp, few_query_rows=64)
    assert vl.tolist() == [1, 1, 1, 1] and idx[:, 0].tolist() == [0, 0, 0, 0]


def test_few_query_more_than_1024_candidate_batches():
    """A row of 4.5M keys has more than 1,024 candidate batches of 256 keys,
    so the cut kernel gathers the candidates in several rounds; ties on
    repeated keys make the rounds' boundaries matter (and may overflow the
    candidate list, which sends the row to the repair launch)."""
    g = torch.Generator().manual_seed(9)
    T, H, d = 4_500_000, 4, 32
    base = torch.randn(4096, d, generator=g)
    k = base[torch.randint(0, 4096, (T,), generator=g)].bfloat16()   # many equal scores
    q = torch.randn(2, H, d, generator=g).bfloat16()
    w = torch.randn(H, generator=g)
    inp = replace(gen.custom(q=q, k=k, w=w, topk=300), q_pos0=T - 2).to(DEV)
    dense, stream = _both_paths(inp)
    _assert_identical(dense, stream)
    assert (dense[1] == 300).all()


def _sample_places(P):
    """Keys of the few-query estimate's sample for a row of P > 8192 keys:
    64 consecutive keys at each of 128 places g * (P - 64) // 127."""
    sp = (P - 64) // 127
    return (np.arange(128)[:, None] * sp + np.arange(64)[None, :]).ravel()


def _adversarial_keys(T, P, kind, g):
    """Column 0 of the keys, read by a query (1, 0, ...) with weight 1, so a
    key's score is ReLU(k[j, 0]).  'high': the sampled keys score 5..15 and
    every other key below 5, so the estimate (a high quantile of the sample)
    leaves fewer candidates than the selection needs; 'overflow': the
    sampled keys tie at 10 and 3,000 other keys score 20, so more keys than
    the candidate list holds reach the estimate.  Column 1 is random."""
    k = torch.zeros(T, 32)
    k[:, 1] = torch.randn(T, generator=g)
    places = torch.from_numpy(_sample_places(P))
    if kind == "high":
        k[:, 0] = 4.0 + torch.arange(T, dtype=torch.float32) / (4 * T)
        k[places, 0] = 5.0 + 10.0 * torch.randperm(places.numel(), generator=g).float() / places.numel()
    else:
        k[:, 0] = 1.0
        k[places, 0] = 10.0
        others = torch.from_numpy(np.setdiff1d(np.arange(T), _sample_places(P)))
        pick = others[torch.randperm(others.numel(), generator=g)[:3000]]
        k[pick, 0] = 20.0
    return k


@pytest.mark.parametrize("kind", ["high", "overflow"])
@pytest.mark.parametrize("S", [1, 3, 8])
def test_few_query_rows_whose_estimate_fails_are_repaired(kind, S):
    """Rows built so that the sampled estimate fails -- too few candidates
    reach it, or more than the list holds -- are selected by the repair
    launch; in a batch, rows reading column 1 (random scores) are cut from
    their candidates as usual.  Either way the result equals the streaming
    path's bit for bit, and the adversarial rows keep exactly the keys the
    construction fixes."""
    g = torch.Generator().manual_seed(31 + S)
    T = 65536
    k = _adversarial_keys(T, T, kind, g)
    q = torch.zeros(S, 1, 32)
    adv = [t % 2 == 0 or S == 1 for t in range(S)]
    for t in range(S):
        q[t, 0, 0 if adv[t] else 1] = 1.0
    inp = replace(gen.custom(q=q.bfloat16(), k=k.bfloat16(), w=torch.ones(1), topk=2048),
                  q_pos0=T - 1, causal=False).to(DEV)
    import dsa_indexer_score_amd as dsai
    ix = dsai.Indexer(torch.bfloat16, few_query_rows=64, device=DEV)
    ws = torch.empty(ix.workspace_bytes(S, T, 1, 32, 1, 2048), dtype=torch.uint8, device=DEV)
    dense = ix.score_topk(inp.q, inp.w, inp.k, topk=2048, causal=False, with_scores=True,
                          workspace=ws)
    stream = run(inp, few_query_rows=-1)
    _assert_identical(dense, stream)
    # the repair marks, at their documented place in the workspace (after
    # the sample and witness scores, estimates and 32 sub-list counts):
    # exactly the adversarial rows
    up = lambda x: -(-x // 256) * 256
    at = up(S * 16384 * 4) + up(S * 4) + up(S * 32 * 4)
    status = ws[at:at + 4 * S].view(torch.int32).cpu().tolist()
    assert status == [1 if a else 0 for a in adv], status
    kb = k.bfloat16().float()[:, 0]
    want = torch.sort(torch.argsort(-kb, stable=True)[:2048]).values.int()
    for t in range(S):
        if adv[t]:
            assert torch.equal(dense[0][t].cpu(), want), t
    log(f"  {kind} S={S}: adversarial rows {sum(adv)} of {S}")


def test_few_query_rows_in_passes():
    """The no-allocation entry point sizes few-query passes to its 256 MiB
    scratch: 1,500 decode rows at a 1M-token context (262,144 keys, about
    200 KB of candidate lists, directory and sample per row) go in two
    passes of 750, and equal the workspace call's single pass bit for bit."""
    import dsa_indexer_score_amd as dsai
    inp = _decode("c5_csa_1m", 1500, 262144)
    ix = dsai.Indexer(inp.q.dtype, few_query_rows=4096, device=DEV)
    kw = dict(m=inp.m, topk=inp.topk, causal=True, q_scale=inp.q_scale, k_scale=inp.k_scale,
              q_pos0=inp.q_pos0, with_scores=True)
    per_row = ix.workspace_bytes(1, inp.T, inp.H, inp.d, inp.m, inp.topk)
    assert 1500 * per_row > 256 << 20 > 750 * per_row
    ref = ix.score_topk(inp.q, inp.w, inp.k, **kw)
    got = ix.score_topk_noalloc(inp.q, inp.w, inp.k, **kw)
    torch.cuda.synchronize()
    _assert_identical(ref, got)
    assert (ref[1] == 2048).all()
