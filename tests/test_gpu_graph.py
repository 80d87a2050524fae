"""The indexer step under HIP graph capture (torch.cuda.CUDAGraph).

A decode or prefill step launches only kernels on the caller's stream (no
allocation, no memset, no host synchronisation inside the library), so it
can be captured once and replayed.  Each replay is checked against an
eager call on the same inputs, with eager work and synchronisations in
between, and after the inputs change in place.
"""
from dataclasses import replace

import pytest
import torch

from workloads import gen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _capture_and_check(inp, ix, replays=4):
    import dsa_indexer_score_amd as dsai
    W = dsai.output_width(inp.topk, inp.m, inp.expand, inp.tail)
    ws = torch.empty(ix.workspace_bytes(inp.S, inp.T, inp.H, inp.d, inp.m, inp.topk),
                     dtype=torch.uint8, device=DEV)
    idx = torch.empty((inp.S, W), dtype=torch.int32, device=DEV)
    vl = torch.empty((inp.S,), dtype=torch.int32, device=DEV)
    sc = torch.empty((inp.S, W), dtype=torch.float32, device=DEV)
    call = lambda out: ix.score_topk(inp.q, inp.w, inp.k, m=inp.m, topk=inp.topk,
                                     causal=inp.causal, q_scale=inp.q_scale, k_scale=inp.k_scale,
                                     q_pos0=inp.q_pos0, with_scores=True, workspace=ws, out=out)
    call((idx, vl, sc))                                  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call((idx, vl, sc))
    gen_q = torch.Generator(device=DEV).manual_seed(5)
    for r in range(replays):
        if r == replays - 1:                             # new query values, same buffers
            inp.q.copy_((torch.randn(inp.q.shape, generator=gen_q, device=DEV) /
                         inp.d ** 0.5).to(inp.q.dtype))
        g.replay()
        torch.cuda.synchronize()
        ref = ix.score_topk(inp.q, inp.w, inp.k, m=inp.m, topk=inp.topk, causal=inp.causal,
                            q_scale=inp.q_scale, k_scale=inp.k_scale, q_pos0=inp.q_pos0,
                            with_scores=True)
        torch.cuda.synchronize()
        assert torch.equal(ref[0], idx) and torch.equal(ref[1], vl) and torch.equal(ref[2], sc), r


@pytest.mark.parametrize("rows", [1, 5])
def test_decode_step_replays_from_a_graph(rows):
    import dsa_indexer_score_amd as dsai
    T = 65536
    inp = gen.generate("c4_csa_256k", S=rows, T=T)
    inp = replace(inp, q_pos0=T * inp.m - rows, query_chunk=None).to(DEV)
    ix = dsai.Indexer(inp.q.dtype, few_query_rows=64, device=DEV)
    _capture_and_check(inp, ix)


def test_streaming_step_replays_from_a_graph():
    import dsa_indexer_score_amd as dsai
    inp = gen.generate("c4_csa_256k", S=1500, topk=512).to(DEV)
    ix = dsai.Indexer(inp.q.dtype, query_chunk=512, device=DEV)
    _capture_and_check(inp, ix)
