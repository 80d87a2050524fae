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
