"""Witness keys on the few-query path (indexer_score_topk_witness).

"DoSA: Dots Sparse Attention" (summary page, "Method steps", decode): keys
selected at an earlier step serve as witnesses; the Ksel-th best of their
exact scores cannot exceed the row's Ksel-th best score, so it can only
raise the threshold estimate safely.  The selection must not depend on the
witnesses: every case is compared bit for bit with the plain call
(indices, valid lengths, reported scores).  The estimates, candidate counts
and repair marks are read back from the documented few-query workspace
layout to check that the witnesses were used where they can be, ignored
where they cannot, and that a too-high bound (repeated witnesses) is caught
by the exact cut and repaired.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from gpu_util import log
from workloads import gen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _up(x, a=256):
    return -(-x // a) * a


def _pair(name, S, T, rho=None, topk=None):
    """S + 1 rows at the end of a T-key context: row 0 is the previous step
    of row 1, and so on."""
    over = {} if rho is None else {"rho": rho}
    inp = gen.generate(name, S=S + 1, T=T, topk=topk, **over)
    return replace(inp, q_pos0=T * inp.m - (S + 1)).to(DEV)


def _rows(inp, lo, hi):
    return replace(inp, q=inp.q[lo:hi].contiguous(), S=hi - lo, q_pos0=inp.q_pos0 + lo,
                   q_scale=None if inp.q_scale is None else inp.q_scale[lo:hi].contiguous(),
                   w=inp.w if inp.w.dim() == 1 else inp.w[lo:hi].contiguous())


def _indexer(inp, few=64):
    import dsa_indexer_score_amd as dsai
    return dsai.Indexer(inp.q.dtype, expand=inp.expand, tail=inp.tail, few_query_rows=few,
                        device=DEV)


def _call(ix, inp, witness=None):
    """One call with a workspace of its own; returns the outputs and the
    workspace's estimates, candidate totals and repair marks."""
    ws = torch.empty(ix.workspace_bytes(inp.S, inp.T, inp.H, inp.d, inp.m, inp.topk),
                     dtype=torch.uint8, device=DEV)
    out = ix.score_topk(inp.q, inp.w, inp.k, m=inp.m, topk=inp.topk, causal=inp.causal,
                        q_scale=inp.q_scale, k_scale=inp.k_scale, q_pos0=inp.q_pos0,
                        with_scores=True, workspace=ws, witness=witness)
    torch.cuda.synchronize()
    S = inp.S
    b = ws.cpu().numpy()
    est_at = _up(S * 16384 * 4)
    cnt_at = est_at + _up(S * 4)
    stat_at = cnt_at + _up(S * 32 * 4)
    est = np.frombuffer(b[est_at:est_at + 4 * S].tobytes(), np.uint32)
    tot = np.frombuffer(b[cnt_at:cnt_at + 128 * S].tobytes(), np.uint32).reshape(S, 32).sum(1)
    stat = np.frombuffer(b[stat_at:stat_at + 4 * S].tobytes(), np.int32)
    return out, est, tot, stat


def _same(a, b):
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _ksel(inp):
    return inp.topk // inp.m if inp.expand else inp.topk


CASES = [
    ("c5_csa_1m", 1, 262144, None),      # fp8 compressed keys, the 1M-token decode row
    ("c5_csa_1m", 4, 262144, 0.995),     # slowly changing queries
    ("c3_dsa_token", 2, 131072, 0.99),   # fp8 token keys (no expansion)
    ("c4_csa_256k", 3, 65536, None),     # bf16, i.i.d. queries
    ("c2_glm_pooled", 2, 8192, None),    # H = 32, expansion + tail (too few keys to sample)
    ("c2_glm_pooled", 2, 65536, None),   # H = 32, expansion + tail, sampled
]


@pytest.mark.parametrize("name,S,T,rho", CASES)
def test_previous_step_witnesses_give_the_same_selection(name, S, T, rho):
    """Witnesses = the previous position's selection (a decode step):
    identical outputs; the estimate is never lowered."""
    pair = _pair(name, S, T, rho)
    ix = _indexer(pair)
    prev, cur = _rows(pair, 0, S), _rows(pair, 1, S + 1)
    wit = _call(ix, prev)[0][0]
    plain, est0, tot0, _ = _call(ix, cur)
    wout, est1, tot1, _ = _call(ix, cur, witness=wit)
    _same(plain, wout)
    assert np.all(est1 >= est0)
    log(f"  {name} S={S} rho={rho}: estimate raised on {int((est1 > est0).sum())}/{S} rows, "
        f"candidates {tot0.tolist()} -> {tot1.tolist()}")


@pytest.mark.parametrize("name,T", [("c5_csa_1m", 262144), ("c3_dsa_token", 131072),
                                    ("c4_csa_256k", 65536), ("c2_glm_pooled", 65536)])
def test_exact_witnesses_leave_only_the_selection(name, T):
    """Witnesses = the row's own selection: their Ksel-th best is the row's
    Ksel-th best, so the candidates are exactly the selection (no ties on
    continuous data) and no row is repaired."""
    inp = _rows(_pair(name, 3, T), 1, 4)
    ix = _indexer(inp)
    plain, est0, tot0, _ = _call(ix, inp)
    wout, est1, tot1, stat = _call(ix, inp, witness=plain[0])
    _same(plain, wout)
    assert np.all(est1 > est0)
    assert np.all(tot1 == _ksel(inp)) and np.all(tot0 > _ksel(inp))
    assert np.all(stat == 0)


@pytest.mark.parametrize("name,T", [("c5_csa_1m", 262144), ("c2_glm_pooled", 65536)])
def test_witnesses_that_cannot_bound_change_nothing(name, T):
    """No entries, entries naming no visible key (-1, keys or positions past
    the row's, positions other than a pool's first) and fewer than Ksel
    valid witnesses leave the sampled estimate as it is."""
    inp = _rows(_pair(name, 2, T), 1, 3)
    ix = _indexer(inp)
    plain, est0, tot0, _ = _call(ix, inp)
    W = plain[0].shape[1]
    per = inp.m if inp.expand else 1           # entries per selected key
    past = inp.T * per                         # no row sees key T (or its positions)
    g = torch.Generator(device=DEV).manual_seed(3)
    bad = [
        torch.full((inp.S, W), -1, dtype=torch.int32, device=DEV),
        torch.randint(past, past + 3, (inp.S, W), generator=g, device=DEV, dtype=torch.int32),
        plain[0][:, :per * 100].contiguous(),                  # 100 keys < Ksel
        torch.empty((inp.S, 0), dtype=torch.int32, device=DEV),
    ]
    if inp.expand:                                              # never a pool's first position
        bad.append(torch.where(plain[0] >= 0, plain[0] - plain[0] % inp.m + 1, plain[0]))
    for i, wit in enumerate(bad):
        wout, est1, tot1, stat = _call(ix, inp, witness=wit)
        _same(plain, wout)
        assert np.array_equal(est1, est0), i
        assert np.array_equal(tot1, tot0), i


@pytest.mark.parametrize("name,T", [("c5_csa_1m", 262144), ("c2_glm_pooled", 65536)])
def test_repeated_witnesses_are_caught_and_repaired(name, T):
    """Ksel copies of the row's best key (pool): the bound is its score, far
    above the true Ksel-th best; the cut finds one candidate, marks the row,
    and the repair launch gives the exact selection."""
    inp = _rows(_pair(name, 2, T), 1, 3)
    ix = _indexer(inp)
    plain, est0, _, _ = _call(ix, inp)
    idx, sc = plain[0], plain[2]
    ksel = _ksel(inp)
    pos = torch.arange(inp.S, device=DEV)[:, None] + inp.q_pos0
    pooled = (idx >= 0) & (idx < (pos + 1) // inp.m * inp.m)    # not padding, not the tail
    best = torch.argmax(torch.where(pooled, sc, torch.full_like(sc, -torch.inf)), dim=1)
    top = idx.gather(1, best[:, None])
    if inp.expand:
        top = top - top % inp.m                 # the pool's first position
    wit = top.repeat(1, ksel).contiguous()
    wout, est1, tot1, stat = _call(ix, inp, witness=wit)
    _same(plain, wout)
    assert np.all(est1 > est0) and np.all(stat == 1) and np.all(tot1 < ksel)


def test_witness_entries_past_8192_are_not_read():
    """Only the first 8,192 entries of a row's witnesses are scored: with
    those all -1 and the row's own selection after them, the estimate stays
    the sampled one (with the selection within the first 8,192 it would
    become the exact Ksel-th code)."""
    inp = _rows(_pair("c5_csa_1m", 2, 262144), 1, 3)
    ix = _indexer(inp)
    plain, est0, tot0, _ = _call(ix, inp)
    sel = plain[0]
    W = sel.shape[1]
    late = torch.full((inp.S, 8192 + W), -1, dtype=torch.int32, device=DEV)
    late[:, 8192:] = sel
    wout, est1, tot1, _ = _call(ix, inp, witness=late.contiguous())
    _same(plain, wout)
    assert np.array_equal(est1, est0) and np.array_equal(tot1, tot0)
    early = late.clone()
    early[:, :W] = sel
    _, est2, _, _ = _call(ix, inp, witness=early.contiguous())
    assert np.all(est2 > est0)


def test_streaming_path_ignores_witnesses():
    """Rows beyond the few-query limit stream; the witnesses change nothing."""
    inp = _rows(_pair("c4_csa_256k", 40, 4096), 1, 41)
    ix = _indexer(inp, few=-1)
    import dsa_indexer_score_amd as dsai
    W = dsai.output_width(inp.topk, inp.m, inp.expand, inp.tail)
    wit = torch.zeros((inp.S, W), dtype=torch.int32, device=DEV)
    ws = torch.empty(ix.workspace_bytes(inp.S, inp.T, inp.H, inp.d, inp.m, inp.topk),
                     dtype=torch.uint8, device=DEV)
    kw = dict(m=inp.m, topk=inp.topk, causal=inp.causal, q_scale=inp.q_scale,
              k_scale=inp.k_scale, q_pos0=inp.q_pos0, with_scores=True, workspace=ws)
    a = ix.score_topk(inp.q, inp.w, inp.k, **kw)
    b = ix.score_topk(inp.q, inp.w, inp.k, witness=wit, **kw)
    torch.cuda.synchronize()
    _same(a, b)
