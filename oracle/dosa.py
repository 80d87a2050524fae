"""DoSA per-key score certificates (fp64) -- TEST INFRASTRUCTURE ONLY.

"DoSA: Dots Sparse Attention" (summary page, sections "Core method" and
"Method steps"): a key whose score upper bound U_i lies below a lower bound
tau of the row's K-th best score cannot enter the top-K, so its full score
need not be computed.  The construction, step by step:

  1. seed: exact scores of a visible seed set S with |S| >= K; tau is its
     K-th best score (any such subset's K-th best is <= the full set's,
     "Prerequisites: Top-K threshold and subset lower bound").
  2. head budget r: if the positive heads number at most r, keep all of them
     and fill the budget with negative heads in order of
     |w_h| ||q_h|| min(p_h, 1 - p_h), p_h = the head's activation frequency
     (share of seed keys with q_h . k > 0); otherwise keep the r positive
     heads with the largest w_h ||q_h||.
  3. certificate: each omitted positive head h gets an anchor j among the
     kept positive heads, beta_h = [q_h . q_j]_+ / ||q_j||^2 and residual
     d_h = q_h - beta_h q_j, so that [q_h . k]_+ <= beta_h [q_j . k]_+ +
     ||d_h|| ||k|| (ReLU subadditivity and positive homogeneity,
     Cauchy-Schwarz); the anchors' weights fold to w_j + sum_h w_h beta_h
     and the residual allowance is E = sum_h w_h ||d_h||.  The omitted
     negative heads contribute at most -[a_A . k]_+ with a_A =
     sum_{h in A} |w_h| q_h over A = {omitted negative h : p_h >= 1/2}
     (subadditivity: [a_A . k]_+ <= sum_{h in A} |w_h| [q_h . k]_+); the other
     omitted negative heads are dropped (they only lower the score).
     U_i = sum_{kept h} w~_h [q_h . k_i]_+ + E ||k_i|| - [a_A . k_i]_+.
  4. joint residual bound ("Technical novelty"): with u_h = w_h d_h over the
     omitted positive heads, sum_h [u_h . k]_+ <= E_joint ||k|| where
     E_joint = (||sum_h u_h|| + sqrt(sum_{h,l} |u_h . u_l|)) / 2, because
     [x]_+ = (x + |x|) / 2, sum_h u_h . k <= ||sum_h u_h|| ||k|| and
     sum_h |u_h . k| = (sum_h sign_h u_h) . k, whose squared norm factor is
     at most sum_{h,l} |u_h . u_l|.  E_joint <= E (triangle inequality), so
     it replaces E in U_i.

Choices the page leaves open, and the reading taken: the anchor of an
omitted positive head is the kept positive head maximising
[q_h . q_j]_+ / ||q_j|| (the one that removes the most of q_h); when no
positive head is kept the omitted positive heads are bounded by
w_h ||q_h|| ||k|| alone; the seed set is supplied by the caller, and with
an empty seed set every activation frequency p_h is taken as 1/2 (the
negative-head priority is then |w_h| ||q_h|| / 2) and no omitted negative
head counts as majority-active (the aggregate a_A is zero).  u_h carries the
head weight (w_h > 0), so E_joint is in the units of the score.
"""
from __future__ import annotations

import numpy as np


def seed_threshold(scores_seed: np.ndarray, K: int) -> float:
    """tau = K-th best exact score of the seed set (needs |S| >= K)."""
    s = np.sort(np.asarray(scores_seed, np.float64))[::-1]
    if s.size < K:
        raise ValueError("the seed set must hold at least K keys")
    return float(s[K - 1])


def certificate(q: np.ndarray, w: np.ndarray, seed_keys: np.ndarray, r: int, p=None):
    """Certificate of one query: q [H, d], w [H] (fp64), seed_keys [n, d].
    Returns dict(kept, w_fold, E, E_joint, aA, A, p) with U(k) = sum_kept
    w_fold [q k]_+ + E_joint ||k|| - [aA k]_+ (E in place of E_joint gives
    the looser per-head allowance).  p, when given, replaces the activation
    frequencies measured on the seeds (which must then be non-empty): a
    sign decided in another precision may differ for a dot product next to
    zero, and the rest of the construction is then compared on equal
    footing."""
    q = np.asarray(q, np.float64)
    w = np.asarray(w, np.float64)
    H = q.shape[0]
    X = q @ np.asarray(seed_keys, np.float64).T
    # no seed keys: no activation statistics, every p_h taken as 1/2
    if p is not None:
        if not X.shape[1]:
            raise ValueError("activation frequencies come from a non-empty seed set")
        p = np.asarray(p, np.float64)
    else:
        p = (X > 0).mean(axis=1) if X.shape[1] else np.full(H, 0.5)
    norms = np.linalg.norm(q, axis=1)
    pos = [h for h in range(H) if w[h] > 0]
    neg = [h for h in range(H) if w[h] < 0]
    if len(pos) <= r:
        kept = list(pos)
        pri = {h: abs(w[h]) * norms[h] * min(p[h], 1 - p[h]) for h in neg}
        kept += sorted(neg, key=lambda h: -pri[h])[:r - len(pos)]
    else:
        kept = sorted(pos, key=lambda h: -(w[h] * norms[h]))[:r]
    w_fold = {h: float(w[h]) for h in kept}
    kept_pos = [h for h in kept if w[h] > 0]
    E = 0.0
    U_res = []                      # weighted residuals u_h = w_h d_h
    for h in (h for h in pos if h not in kept):
        if kept_pos:
            j = max(kept_pos, key=lambda j: max(q[h] @ q[j], 0.0) / norms[j])
            beta = max(q[h] @ q[j], 0.0) / (q[j] @ q[j])
            w_fold[j] += w[h] * beta
            d_h = q[h] - beta * q[j]
        else:
            d_h = q[h]
        E += w[h] * np.linalg.norm(d_h)
        U_res.append(w[h] * d_h)
    U_res = np.array(U_res).reshape(-1, q.shape[1])
    E_joint = 0.5 * (np.linalg.norm(U_res.sum(axis=0)) + np.sqrt(np.abs(U_res @ U_res.T).sum()))
    # the majority-active set needs activation evidence: empty without seeds
    A = [h for h in neg if h not in kept and p[h] >= 0.5] if X.shape[1] else []
    aA = np.zeros(q.shape[1])
    for h in A:
        aA += abs(w[h]) * q[h]
    return dict(kept=kept, w_fold=np.array([w_fold[h] for h in kept]), E=float(E),
                E_joint=float(E_joint), aA=aA, A=A, p=p, q_kept=q[kept])


def upper_bounds(cert: dict, keys: np.ndarray, joint: bool = True) -> np.ndarray:
    """U_i for every key row of keys [n, d] (fp64); joint=False uses the
    per-head allowance E instead of E_joint."""
    keys = np.asarray(keys, np.float64)
    Xk = cert["q_kept"] @ keys.T
    E = cert["E_joint"] if joint else cert["E"]
    return (cert["w_fold"] @ np.maximum(Xk, 0.0) + E * np.linalg.norm(keys, axis=1)
            - np.maximum(keys @ cert["aA"], 0.0))
