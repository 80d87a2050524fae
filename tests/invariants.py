"""Checks that hold for every output row of the indexer, at any size.

Visibility and width follow GLM-5.3-Flash Module 06 "DSA & KPool"
(sections 2-3); the ascending order follows "Adjacent-Query KV-Index Overlap
in 256K DSA Training" (section 3: indices sorted by KV index).
"""
import numpy as np

from oracle import oracle as orc


def check_rows(idx, valid_len, rows, *, T, m, topk, causal, expand, tail, q_pos0=0):
    """idx [n, W] int, valid_len [n] for absolute rows ``rows`` (indices into
    the call's queries).  Raises AssertionError naming the first bad row."""
    idx = np.asarray(idx)
    valid_len = np.asarray(valid_len)
    W = orc.output_width(topk, m, expand, tail)
    assert idx.shape[1] == W, (idx.shape, W)
    for r, t in enumerate(rows):
        p = int(t) + q_pos0
        v = int(valid_len[r])
        ev = orc.expected_valid_len(p, T, m, topk, causal, expand, tail)
        assert v == ev, f"row {t}: valid_len {v} != {ev}"
        row = idx[r]
        assert np.all(row[v:] == -1), f"row {t}: padding not -1"
        sel = row[:v]
        assert np.all(sel >= 0), f"row {t}: negative index"
        assert np.all(np.diff(sel) > 0), f"row {t}: not strictly ascending"
        if v:
            if expand:
                lim = (p + 1) if causal else T * m
            else:
                lim = orc.visible_keys(p, T, m, causal)
            assert sel[-1] < lim, f"row {t}: index {sel[-1]} not visible (limit {lim})"
        if expand and v:
            P = orc.visible_keys(p, T, m, causal)
            body = sel[sel < P * m] if causal else sel
            # every selected pool contributes all m of its positions
            assert body.size % m == 0, f"row {t}: partial pool"
            pools = body.reshape(-1, m)
            assert np.all(pools == pools[:, :1] + np.arange(m)), f"row {t}: pool not contiguous"
            assert np.all(pools[:, 0] % m == 0), f"row {t}: pool not aligned"
    return True
