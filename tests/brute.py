"""Brute-force reference for tiny problems, independent of the C oracle.

Scores come from numpy matrix products in fp64 (a library routine), and the
selection uses no sort at all: key j is selected iff fewer than Ksel keys
beat it, where j' beats j when s_j' > s_j, or s_j' == s_j and j' < j.
Inputs are already-dequantised fp64 arrays.
"""
import numpy as np


def brute_row(Qt, wt, K, p, T, m, topk, causal, expand, tail):
    """Qt [H, d], wt [H], K [T, d] (fp64).  Returns (row indices ascending,
    selected key set, fp64 scores of the visible keys)."""
    P = T if not causal else min(T, (p + 1) // m)
    Ksel = topk // m if expand else topk
    X = Qt @ K[:P].T                                  # [H, P]
    s = wt @ np.maximum(X, 0.0)                        # [P]
    beats = (s[None, :] > s[:, None]) | ((s[None, :] == s[:, None]) &
                                         (np.arange(P)[None, :] < np.arange(P)[:, None]))
    rank = beats.sum(axis=1)                           # how many keys beat key j
    sel = np.nonzero(rank < Ksel)[0]
    if expand:
        pos = (sel[:, None] * m + np.arange(m)[None, :]).ravel()
        if tail and causal:
            pos = np.concatenate([pos, np.arange(P * m, p + 1)])
    else:
        pos = sel
    return np.sort(pos), set(sel.tolist()), s


def dequant(inp):
    """IndexerInputs -> fp64 numpy (Q [S,H,d], W [S,H], K [T,d]) via torch's
    own casts (bf16 / float8_e4m3fn -> float32 are library conversions)."""
    q = inp.q.detach().cpu().float().double().numpy()
    k = inp.k.detach().cpu().float().double().numpy()
    if inp.q_scale is not None:
        q = q * inp.q_scale.detach().cpu().double().numpy()[:, :, None]
    if inp.k_scale is not None:
        k = k * inp.k_scale.detach().cpu().double().numpy()[:, None]
    w = inp.w.detach().cpu().double().numpy()
    if w.ndim == 1:
        w = np.broadcast_to(w, (inp.S, inp.H))
    return q, w, k
