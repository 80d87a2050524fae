"""The few-query path (dense scores + candidate filter + exact cut per row)
against the streaming path and the oracle.

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


def test_few_query_more_than_1024_candidate_segments():
    """A row of 4.5M keys has more than 1,024 filter segments of 4,096 keys,
    so the cut kernel gathers the candidates in several rounds; ties on
    repeated keys make the rounds' boundaries matter."""
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


def test_few_query_rows_in_passes():
    """Eight decode rows over 48M keys need more than the 4 GiB the dense
    workspace may take, so the rows go in two equal passes (4 + 4; 7 would
    fit); each row equals the same row scored and cut on its own."""
    import dsa_indexer_score_amd as dsai
    g = torch.Generator().manual_seed(21)
    S, T, H, d = 8, 48_000_000, 4, 32
    base = (torch.randn(1 << 16, d, generator=g) / d ** 0.5).bfloat16()
    k = base[torch.randint(0, 1 << 16, (T,), generator=g)].to(DEV)
    q = (torch.randn(S, H, d, generator=g) / d ** 0.5).bfloat16().to(DEV)
    w = torch.randn(S, H, generator=g).to(DEV)
    kw = dict(m=1, topk=700, causal=True, few_query_rows=64, with_scores=True)
    h = dsai.Indexer(torch.bfloat16, few_query_rows=64, device=DEV)
    assert 6 * 12 * T < h.workspace_bytes(S, T, H, d, 1, 700) <= 1 << 32   # 7 rows a pass
    idx, vl, sc = dsai.score_topk(q, w, k, q_pos0=T - S, **kw)
    torch.cuda.synchronize()
    for t in range(S):
        i1, v1, s1 = dsai.score_topk(q[t:t + 1].contiguous(), w[t:t + 1].contiguous(), k,
                                     q_pos0=T - S + t, **kw)
        torch.cuda.synchronize()
        assert torch.equal(i1[0], idx[t]) and torch.equal(v1[0], vl[t]), t
        assert torch.equal(s1[0], sc[t]), t
    assert (vl == 700).all()
