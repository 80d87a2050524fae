"""The no-allocation entry point (indexer_score_topk_noalloc) against the
workspace entry point it varies (indexer_score_topk), through the C ABI:
same kernels, so every output must be identical bit for bit -- including
where the static scratch forces other launch sizes than the workspace call
uses.  Each case makes two calls in a row, the second on a smaller input,
since the scratch keeps the previous call's contents."""
from dataclasses import replace

import pytest
import torch

from gpu_util import log
from workloads import gen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair(inp, **handle):
    """(workspace call, no-allocation call) outputs of one problem."""
    import dsa_indexer_score_amd as dsai
    ix = dsai.Indexer(inp.q.dtype, expand=inp.expand, tail=inp.tail, device=DEV, **handle)
    kw = dict(m=inp.m, topk=inp.topk, causal=inp.causal, q_scale=inp.q_scale,
              k_scale=inp.k_scale, q_pos0=inp.q_pos0, with_scores=True)
    ref = ix.score_topk(inp.q, inp.w, inp.k, **kw)
    W = dsai.output_width(inp.topk, inp.m, inp.expand, inp.tail)
    out = (torch.full((inp.S, W), -7, dtype=torch.int32, device=DEV),
           torch.full((inp.S,), -7, dtype=torch.int32, device=DEV),
           torch.full((inp.S, W), -7.0, dtype=torch.float32, device=DEV))
    got = ix.score_topk_noalloc(inp.q, inp.w, inp.k, out=out, **kw)
    torch.cuda.synchronize()
    return ref, got


def _same(ref, got, what):
    for a, b, name in zip(ref, got, ("idx", "valid_len", "sel_score")):
        assert torch.equal(a, b), f"{what}: {name} differs"


def _end_of_context(name, S, T, **kw):
    inp = gen.generate(name, S=S, T=T, **kw)
    return replace(inp, q_pos0=T * inp.m - S).to(DEV)


CASES = [
    # streaming, launches sized to the scratch (20,736 candidate slots per
    # row: 1,616 rows per launch instead of one launch of all rows)
    ("c4 end of context", lambda: _end_of_context("c4_csa_256k", 4100, 65536),
     lambda: _end_of_context("c4_csa_256k", 1500, 40000), {"few_query_rows": -1}),
    # streaming with expansion and tail, fp8 with scales, query chunks
    ("c2 pooled", lambda: gen.generate("c2_glm_pooled", S=3000).to(DEV),
     lambda: gen.generate("c2_glm_pooled", S=700).to(DEV), {}),
    ("c3 fp8", lambda: gen.generate("c3_dsa_token", S=2500).to(DEV),
     lambda: gen.generate("c3_dsa_token", S=1200).to(DEV), {"query_chunk": 1024}),
    # few-query path (decode rows at the end of a 1M-token context)
    ("c5 decode", lambda: _end_of_context("c5_csa_1m", 3, 262144),
     lambda: _end_of_context("c5_csa_1m", 1, 131072), {}),
    # integer-exact problem, where results are unique
    ("c1 integers", lambda: gen.generate("c1_tiny_int").to(DEV),
     lambda: gen.generate("c1_tiny_int", S=300).to(DEV), {}),
]


@pytest.mark.parametrize("what,big,small,handle", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_workspace_call(what, big, small, handle):
    for n, make in enumerate((big, small)):
        inp = make()
        log(f"  {what} call {n}: S={inp.S} T={inp.T} dtype={inp.dtype} q_pos0={inp.q_pos0}")
        ref, got = _pair(inp, **handle)
        _same(ref, got, f"{what} call {n}")
