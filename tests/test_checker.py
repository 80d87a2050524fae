"""The parity checker accepts the oracle's own rows and rejects planted
mistakes (all on the CPU, mistakes planted into copies of oracle output)."""
import numpy as np

from oracle import check
from oracle import oracle as orc
from workloads import gen


def _scores_for(inp, rows, out):
    """Per-slot fp32 scores as a kernel would report them."""
    W = out["idx"].shape[1]
    sel = np.zeros((len(rows), W), np.float32)
    for r, t in enumerate(rows):
        n = out["n_sel"][r]
        sc = dict(zip(out["key_idx"][r][:n].tolist(), out["key_score"][r][:n].tolist()))
        P = orc.visible_keys(int(t), inp.T, inp.m, inp.causal)
        for i in range(out["valid_len"][r]):
            pos = int(out["idx"][r][i])
            if inp.expand:
                if pos < P * inp.m:
                    sel[r, i] = sc[pos // inp.m]
            else:
                sel[r, i] = sc[pos]
    return sel


def test_checker_accepts_oracle_rows_and_rejects_mistakes():
    inp = gen.generate("c2_glm_pooled", S=200, topk=32)
    rows = np.arange(inp.S)
    out = orc.select_rows(inp, rows)
    sel = _scores_for(inp, rows, out)
    rep = check.compare(inp, rows, out["idx"], out["valid_len"], sel, ref=out)
    assert rep["ok"], rep["failures"]
    # swap a selected pool for a clearly worse visible one
    t = 150
    bad = out["idx"].copy()
    P = orc.visible_keys(t, inp.T, inp.m, True)
    chosen = set(out["key_idx"][t][:out["n_sel"][t]].tolist())
    worst = min((j for j in range(P) if j not in chosen),
                key=lambda j: orc.pair_scores(inp, [t], [j])[0])
    keys = sorted((chosen - {out["key_idx"][t][0]}) | {worst})
    body = np.concatenate([np.arange(j * 4, j * 4 + 4) for j in keys])
    tl = bad[t][len(body):out["valid_len"][t]]
    bad[t][:out["valid_len"][t]] = np.concatenate([body, tl])
    rep = check.compare(inp, rows, bad, out["valid_len"], None, ref=out)
    assert not rep["ok"]
    # a wrong length
    vl = out["valid_len"].copy()
    vl[7] += 1
    assert not check.compare(inp, rows, out["idx"], vl, None, ref=out)["ok"]
    # a score off by more than the tolerance
    sel2 = sel.copy()
    sel2[100, 0] *= 1.01
    assert not check.compare(inp, rows, out["idx"], out["valid_len"], sel2, ref=out)["ok"]


def test_checker_exact_mode_is_bit_exact():
    inp = gen.generate("c1_tiny_int", S=128)
    rows = np.arange(inp.S)
    out = orc.select_rows(inp, rows)
    sel = _scores_for(inp, rows, out)
    assert check.compare(inp, rows, out["idx"], out["valid_len"], sel, ref=out)["ok"]
    sel[90, 3] += 0.5
    assert not check.compare(inp, rows, out["idx"], out["valid_len"], sel, ref=out)["ok"]
    bad = out["idx"].copy()
    bad[120, 0] += 0  # unchanged row passes; a changed index fails
    bad[121, 5] = bad[121, 5] + 1 if bad[121, 5] + 1 not in bad[121] else bad[121, 5]
    if not np.array_equal(bad, out["idx"]):
        assert not check.compare(inp, rows, bad, out["valid_len"], None, ref=out)["ok"]


def test_sample_rows_cover_boundaries():
    rows = check.sample_rows(262144, m=4, ksel=2048, chunk=16384, n_uniform=64)
    for r in (0, 3, 4, 2047, 2048, 8191, 8192, 16383, 16384, 16385, 262143):
        assert r in rows


def _mutants(inp, out, t):
    """Malformed copies of output row t (duplicate, swap, invisible index,
    broken pool, partial pool, bad padding, wrong tail), each named."""
    v = int(out["valid_len"][t])
    row = out["idx"][t].copy()
    P = orc.visible_keys(int(t) + inp.q_pos0, inp.T, inp.m, inp.causal)
    res = {}
    r = row.copy(); r[v - 1] = r[v - 2]; res["duplicate"] = r
    r = row.copy(); r[[0, inp.m]] = r[[inp.m, 0]]; res["swap"] = r
    short = next(u for u in range(out["idx"].shape[0]) if 1 < out["valid_len"][u] < row.size)
    r = out["idx"][short].copy(); r[out["valid_len"][short]] = 0; res["padding"] = (short, r)
    if inp.expand:
        # replace one selected pool by an unselected visible pool, but move one
        # of its positions (pool no longer whole / aligned)
        r = row.copy(); r[1] = r[1] + 1 if r[1] + 1 != r[2] else r[1]; r[2] = r[1] + 5
        res["broken_pool"] = np.concatenate([np.sort(r[:v]), r[v:]])
        body = row[row < P * inp.m]
        r = row.copy(); r[body.size - 1] = -1
        r[:v] = np.concatenate([np.sort(r[:v][r[:v] >= 0]), [-1]])[:v]
        res["partial_pool"] = r
        r = row.copy(); r[v - 1] = r[v - 1] + 1; res["wrong_tail"] = r
        r = row.copy(); r[v - 1] = int(t) + inp.q_pos0 + 1; res["invisible"] = r
    else:
        r = row.copy(); r[v - 1] = P; res["invisible"] = r
    return res


def test_checker_rejects_malformed_rows_float_mode():
    """Rows that are not valid outputs fail even when every key they name is
    a correct one: repeated entries, order, padding, visibility, pools and
    the tail are checked on every row, not only the scores."""
    for name, S, topk in (("c2_glm_pooled", 200, 32), ("c4_csa_256k", 400, 40),
                          ("c3_dsa_token", 300, 48)):
        inp = gen.generate(name, S=S, topk=topk)
        rows = np.arange(inp.S)
        out = orc.select_rows(inp, rows)
        sel = _scores_for(inp, rows, out)
        assert check.compare(inp, rows, out["idx"], out["valid_len"], sel, ref=out)["ok"]
        t = inp.S - 3
        for what, mrow in _mutants(inp, out, t).items():
            u, mrow = mrow if isinstance(mrow, tuple) else (t, mrow)
            assert not np.array_equal(mrow, out["idx"][u]), (name, what)
            bad = out["idx"].copy()
            bad[u] = mrow
            for with_scores in (True, False):
                rep = check.compare(inp, rows, bad, out["valid_len"],
                                    sel if with_scores else None, ref=out)
                assert not rep["ok"], (name, what)


def test_checker_rejects_malformed_rows_exact_mode():
    inp = gen.generate("c1_tiny_int", S=128)
    rows = np.arange(inp.S)
    out = orc.select_rows(inp, rows)
    t = 100
    for what, mrow in _mutants(inp, out, t).items():
        u, mrow = mrow if isinstance(mrow, tuple) else (t, mrow)
        bad = out["idx"].copy()
        bad[u] = mrow
        assert not check.compare(inp, rows, bad, out["valid_len"], None, ref=out)["ok"], what


def test_row_structure_names_each_problem():
    kw = dict(T=8, m=4, topk=8, causal=True, expand=True, tail=True)
    # position 9: pools 0 and 1 complete (P = 2), tail 8, 9 -> valid_len 10
    good = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 9, -1])
    assert check.row_structure(good, 10, 9, **kw) == []
    assert check.row_structure(np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, -1, -1]), 9, 9, **kw)
    assert check.row_structure(np.array([0, 1, 2, 3, 4, 5, 7, 6, 8, 9, -1]), 10, 9, **kw)
    assert check.row_structure(np.array([1, 2, 3, 4, 5, 6, 7, 8, 8, 9, -1]), 10, 9, **kw)
    assert check.row_structure(np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 0]), 10, 9, **kw)
    assert check.row_structure(np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 10, -1]), 10, 9, **kw)
