"""Helpers for the GPU tests: run the HIP path through the C ABI and check
all-row invariants on the device (vectorised torch ops, row blocks)."""
import sys

import numpy as np
import torch

import dsa_indexer_score_amd as dsai


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run(inp, *, with_scores=True, query_chunk=None, **overrides):
    """Run one indexer step for an IndexerInputs already on the GPU."""
    kw = dict(m=inp.m, topk=inp.topk, causal=inp.causal, expand=inp.expand, tail=inp.tail,
              q_scale=inp.q_scale, k_scale=inp.k_scale, q_pos0=inp.q_pos0,
              query_chunk=inp.query_chunk if query_chunk is None else query_chunk,
              with_scores=with_scores)
    # these tests target the streaming path unless they name the few-query
    # path (which has tests of its own; the sweeps also run the default)
    kw["few_query_rows"] = -1
    kw.update(overrides)
    out = dsai.score_topk(inp.q, inp.w, inp.k, **kw)
    torch.cuda.synchronize()
    return out


def rows_to_host(rows, *tensors):
    r = torch.as_tensor(np.asarray(rows, np.int64), device=tensors[0].device)
    return [None if t is None else t.index_select(0, r).cpu().numpy() for t in tensors]


def device_invariants(inp, idx, vl, block=16384):
    """valid_len formula, -1 padding, strictly ascending, visibility, for every row."""
    S, W = idx.shape
    dev = idx.device
    m, T = inp.m, inp.T
    ksel = inp.topk // m if inp.expand else inp.topk
    for r0 in range(0, S, block):
        r1 = min(S, r0 + block)
        p = torch.arange(r0, r1, device=dev, dtype=torch.int64) + inp.q_pos0
        if inp.causal:
            P = torch.clamp((p + 1) // m, max=T)
        else:
            P = torch.full_like(p, T)
        if inp.expand:
            tl = (p + 1 - P * m) if (inp.causal and inp.tail) else torch.zeros_like(p)
            ev = torch.clamp(P, max=ksel) * m + tl
            lim = (p + 1) if inp.causal else torch.full_like(p, T * m)
        else:
            ev = torch.clamp(P, max=ksel)
            lim = P
        v = vl[r0:r1].long()
        bad = torch.nonzero(v != ev)
        assert bad.numel() == 0, f"row {r0 + int(bad[0])}: valid_len {int(v[bad[0]])} != {int(ev[bad[0]])}"
        x = idx[r0:r1].long()
        cols = torch.arange(W, device=dev)
        valid = cols[None, :] < v[:, None]
        assert bool(((x == -1) | valid).all()), f"rows {r0}..: padding is not -1"
        assert bool(((x >= 0) | ~valid).all()), f"rows {r0}..: negative index"
        assert bool(((x < lim[:, None]) | ~valid).all()), f"rows {r0}..: index not visible"
        if W > 1:
            both = valid[:, 1:]
            assert bool(((x[:, 1:] > x[:, :-1]) | ~both).all()), f"rows {r0}..: not ascending"
    return True
