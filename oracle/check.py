"""Parity rule between an indexer result and the oracle -- TEST INFRASTRUCTURE.

Integer-exact problems: every index, length and selected score must match
the oracle bit for bit (all sums are exact in fp32 and fp64).

Float problems (bf16: rtol 2e-3; fp8: rtol 1e-3 against the dequantised
fp64 oracle): several top-k sets are correct when scores sit within rounding
of the k-th score, so the unique part is compared exactly and the rest is
checked for validity.

General fp32 inputs (no stated tolerance): the bound of fp32 evaluation is
used instead of a relative tolerance: |s - s*| <= gamma_n * B with
B = sum_h |w_h| sum_i |q_hi k_i|, gamma_n = n u / (1 - n u), u = 2^-24,
n = d + H + 4 (the dot, the head sum and the final products), and keys may
trade places when their oracle scores lie within twice the largest such
bound of the k-th score.

Row structure, checked on every row in both modes before any comparison
(GLM-5.3-Flash Module 06 "DSA & KPool", sections 2-3; "Adjacent-Query
KV-Index Overlap in 256K DSA Training", section 3):
  * valid_len equals the visibility formula; slots from valid_len on are -1;
  * the first valid_len entries are non-negative and strictly ascending, so
    no index repeats;
  * every entry is visible to the row (key < P, or position <= p);
  * in expand mode the entries below P*m form whole pools -- m consecutive
    positions starting at a multiple of m -- and the entries from P*m on are
    exactly the tail positions P*m .. p (none without the tail flag).

Rules for the float problems:
  * valid_len and the tail positions must match exactly;
  * with tau the oracle's k-th score and eps = 1e-3 * max |s*| over the
    oracle's selection (a floor that keeps the rule relative to the row's
    scale where scores cross zero), tol(x) = rtol * max(|x|, eps):
      - every key the result selects but the oracle does not has
        s* >= tau - tol(tau);
      - every key the oracle selects but the result does not has
        s* <= tau + tol(tau);
  * a reported score of a selected key is within tol(s*) of the oracle's.
"""
from __future__ import annotations

import numpy as np

from . import oracle as orc

RTOL = {"bf16": 2e-3, "fp8": 1e-3, "f32": None}
U32 = 2.0 ** -24


def sample_rows(S, *, m=1, ksel=2048, chunk=None, seed=0, n_uniform=256, causal=True):
    """Boundary rows (first rows, m-1/m, K-1/K, K*m-1/K*m, chunk edges +-1,
    last rows) plus seeded uniform rows, clipped to [0, S)."""
    rows = set(range(min(8, S)))
    for r in (m - 1, m, ksel - 1, ksel, ksel * m - 1, ksel * m, ksel * m + 1):
        rows.add(r)
    if chunk:
        for c in range(chunk, S, chunk):
            rows.update((c - 1, c, c + 1))
    rows.update(range(max(0, S - 4), S))
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, S, size=min(n_uniform, S)).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < S), dtype=np.int64)


def row_structure(row, v, p, *, T, m, topk, causal, expand, tail):
    """Problems with one output row (row = its W slots, v = its valid_len,
    p = its absolute position), as a list of strings (empty = well formed)."""
    row = np.asarray(row, np.int64)
    fails = []
    ev = orc.expected_valid_len(p, T, m, topk, causal, expand, tail)
    if v != ev:
        fails.append(f"valid_len {v} != {ev}")
    if v < 0 or v > row.size:
        return fails + [f"valid_len {v} outside the row"]
    if np.any(row[v:] != -1):
        fails.append("padding is not -1")
    sel = row[:v]
    if np.any(sel < 0):
        fails.append("negative index")
    if np.any(np.diff(sel) <= 0):
        fails.append("entries not strictly ascending (repeated or out of order)")
    P = orc.visible_keys(p, T, m, causal)
    if not expand:
        if sel.size and sel.max() >= P:
            fails.append(f"key {int(sel.max())} not visible (P = {P})")
        return fails
    body, tl = sel[sel < P * m], sel[sel >= P * m]
    want_tail = np.arange(P * m, p + 1) if (tail and causal) else np.empty(0, np.int64)
    if not np.array_equal(tl, want_tail):
        fails.append("tail is not exactly the positions P*m .. p")
    if body.size % m:
        fails.append("partial pool")
    else:
        pools = body.reshape(-1, m)
        if np.any(pools != pools[:, :1] + np.arange(m)) or np.any(pools[:, 0] % m):
            fails.append("pool not whole or not aligned")
    return fails


def _keys_of_row(row, v, P, m, expand):
    """Selected keys and the tail part of one output row."""
    sel = np.asarray(row[:v])
    if not expand:
        return sel.astype(np.int64), np.empty(0, np.int64), None
    body = sel[sel < P * m]
    tail = sel[sel >= P * m]
    keys = body[::m] // m if body.size else body
    return keys.astype(np.int64), tail.astype(np.int64), body


def compare(inp, rows, idx, valid_len, sel_score=None, *, exact=None, rtol=None, ref=None,
            nthreads=0):
    """Check result rows (numpy arrays for the given call rows) against the
    oracle.  Returns a report dict; report['ok'] is the outcome and
    report['failures'] lists the first problems found."""
    rows = np.asarray(rows, np.int64)
    idx = np.asarray(idx)
    valid_len = np.asarray(valid_len)
    if exact is None:
        exact = inp.dtype == "f32" and inp.meta.get("qdist") == "int"
    rtol = RTOL[inp.dtype] if rtol is None else rtol
    use_bound = rtol is None and not exact
    nops = inp.d + inp.H + 4
    gamma = nops * U32 / (1 - nops * U32)
    if ref is None:
        ref = orc.select_rows(inp, rows, nthreads=nthreads)
    m, expand = inp.m, inp.expand
    fails = []
    rep = dict(rows=int(rows.size), exact=bool(exact),
               rtol=None if rtol is None else float(rtol), index_mismatch_rows=0,
               extra_keys=0, missing_keys=0, max_score_rel_err=0.0)

    # pass 1: structure, and collect keys that need an oracle score
    need_rows, need_keys, pending = [], [], []
    for r, t in enumerate(rows):
        v = int(valid_len[r])
        bad = row_structure(idx[r], v, int(t) + inp.q_pos0, T=inp.T, m=m, topk=inp.topk,
                            causal=inp.causal, expand=expand, tail=inp.tail)
        if bad:
            fails.extend(f"row {t}: {b}" for b in bad)
            continue
        if v != ref["valid_len"][r]:
            fails.append(f"row {t}: valid_len {v} != {ref['valid_len'][r]}")
            continue
        if exact:
            if not np.array_equal(idx[r], ref["idx"][r]):
                fails.append(f"row {t}: indices differ")
            continue
        p = int(t) + inp.q_pos0
        P = orc.visible_keys(p, inp.T, m, inp.causal)
        G, gtail, _ = _keys_of_row(idx[r], v, P, m, expand)
        O, otail, _ = _keys_of_row(ref["idx"][r], v, P, m, expand)
        if not np.array_equal(gtail, otail):
            fails.append(f"row {t}: tail differs")
        extra = np.setdiff1d(G, O)
        missing = np.setdiff1d(O, G)
        if extra.size or missing.size:
            rep["index_mismatch_rows"] += 1
        pending.append((r, t, G, extra, missing))
        need_rows.extend([r] * G.size)
        need_keys.extend(G.tolist())

    # oracle scores of every key the result selected (extra ones included)
    s_star = b_star = np.empty(0)
    if need_rows:
        s_star = orc.pair_scores(inp, rows[np.asarray(need_rows)], np.asarray(need_keys),
                                 nthreads=nthreads)
        if use_bound:
            b_star = orc.pair_scores(inp, rows[np.asarray(need_rows)], np.asarray(need_keys),
                                     nthreads=nthreads, bounds=True)
    off = 0
    for r, t, G, extra, missing in pending:
        n = int(ref["n_sel"][r])
        okeys = ref["key_idx"][r][:n]
        oscore = ref["key_score"][r][:n]
        tau = float(ref["tau"][r]) if n else 0.0
        eps = 1e-3 * float(np.max(np.abs(oscore))) if n else 0.0
        sg = dict(zip(G.tolist(), s_star[off:off + G.size].tolist()))
        if use_bound:
            bg = dict(zip(G.tolist(), b_star[off:off + G.size].tolist()))
            tol_tau = 2 * gamma * max(bg.values(), default=0.0)
        else:
            tol_tau = rtol * max(abs(tau), eps)
        off += G.size
        so = dict(zip(okeys.tolist(), oscore.tolist()))
        for j in extra.tolist():
            rep["extra_keys"] += 1
            if sg[j] < tau - tol_tau:
                fails.append(f"row {t}: selected key {j} score {sg[j]:.6g} below tau {tau:.6g}")
        for j in missing.tolist():
            rep["missing_keys"] += 1
            if so[j] > tau + tol_tau:
                fails.append(f"row {t}: dropped key {j} score {so[j]:.6g} above tau {tau:.6g}")
        if sel_score is not None and G.size:
            v = int(valid_len[r])
            row = np.asarray(idx[r][:v])
            srow = np.asarray(sel_score[r][:v], np.float64)
            P = orc.visible_keys(int(t) + inp.q_pos0, inp.T, m, inp.causal)
            if expand:
                mask = row < P * m
                keys, got = row[mask][::m] // m, srow[mask][::m]
            else:
                keys, got = row, srow
            want = np.array([sg[int(j)] for j in keys])
            err = np.abs(got - want) / np.maximum(np.abs(want), max(eps, 1e-30))
            rep["max_score_rel_err"] = max(rep["max_score_rel_err"], float(err.max(initial=0)))
            if use_bound:
                lim = gamma * np.array([bg[int(j)] for j in keys])
            else:
                lim = rtol * np.maximum(np.abs(want), eps)
            bad = np.nonzero(np.abs(got - want) > lim)[0]
            if bad.size:
                j = int(keys[bad[0]])
                fails.append(f"row {t}: score of key {j} {got[bad[0]]:.7g} vs {sg[j]:.7g}")

    if exact and sel_score is not None:
        for r, t in enumerate(rows):
            v = int(valid_len[r])
            if v != ref["valid_len"][r]:
                continue
            n = int(ref["n_sel"][r])
            want = dict(zip(ref["key_idx"][r][:n].tolist(), ref["key_score"][r][:n].tolist()))
            mexp = m if expand else 1
            P = orc.visible_keys(int(t) + inp.q_pos0, inp.T, m, inp.causal)
            for i in range(v):
                pos = int(idx[r][i])
                if expand and pos >= P * m:
                    continue
                if float(sel_score[r][i]) != want.get(pos // mexp, np.nan):
                    fails.append(f"row {t}: score at slot {i} not exact")
                    break
    rep["failures"] = fails[:20]
    rep["n_failures"] = len(fails)
    rep["ok"] = not fails
    return rep
