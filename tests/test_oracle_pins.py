"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each test checks it against a
hand-computed worked example (tests/golden/), a closed form, a library
routine, or an independent brute force on tiny inputs.
"""
import numpy as np
import pytest
import torch

from brute import brute_row, dequant
from golden_io import load, scalar
from invariants import check_rows
from oracle import oracle as orc
from workloads import gen


def _we_inputs(rec, S, expand=False, tail=False):
    H, d, m, topk = (scalar(rec, x) for x in ("H", "d", "m", "topk"))
    heads = [[float(v) for v in rec[f"q{h}"][0]] for h in range(H)]
    q = torch.tensor(heads, dtype=torch.float32).expand(S, H, d).contiguous()
    w = torch.tensor([float(v) for v in rec["w"][0]], dtype=torch.float32)
    k = torch.tensor([[float(v) for v in row] for row in rec["k"]], dtype=torch.float32)
    return gen.custom(q=q, k=k, w=w, m=m, topk=topk, causal=True, expand=expand, tail=tail)


def test_we1_scores_and_rows():
    rec = load("we1_signed_relu.txt")
    inp = _we_inputs(rec, S=4)
    want = [float(v) for v in rec["score"][0]]
    got = orc.pair_scores(inp, [3] * 4, [0, 1, 2, 3])
    assert list(got) == want
    out = orc.select_rows(inp, np.arange(4))
    for row in rec["row"]:
        t, v, *ids = (int(x) for x in row)
        assert out["valid_len"][t] == v
        assert list(out["idx"][t]) == ids


def test_we1_pair_overlap():
    rec = load("we1_signed_relu.txt")
    inp = _we_inputs(rec, S=4)
    out = orc.select_rows(inp, np.arange(4))
    shared = orc.pair_overlap(out["idx"], out["valid_len"])
    vl = out["valid_len"]
    for pair in rec["pair"]:
        i, sh, ov, jac = int(pair[0]), int(pair[1]), float(pair[2]), float(pair[3])
        assert shared[i] == sh
        va, vb = vl[2 * i], vl[2 * i + 1]
        assert shared[i] / min(va, vb) == pytest.approx(ov)
        assert shared[i] / (va + vb - shared[i]) == pytest.approx(jac)
    st = orc.overlap_stats(shared, vl)
    assert st["mean_overlap"] == pytest.approx(0.75)
    assert st["mean_jaccard"] == pytest.approx((0.5 + 1 / 3) / 2)


def test_we1_pair_regions():
    """WE1's rows by hand: pair (0,1) = {0} / {0,1}: shared {0}, left {},
    right {1}; pair (2,3) = {0,2} / {0,3}: shared {0}, left {2}, right {3}
    (the three regions of the q-cluster split, Overlap page section 6.1)."""
    rec = load("we1_signed_relu.txt")
    out = orc.select_rows(_we_inputs(rec, S=4), np.arange(4))
    sh, le, ri, cnt = orc.pair_regions(out["idx"], out["valid_len"])
    assert cnt.tolist() == [[1, 0, 1], [1, 1, 1]]
    assert sh[0, :1].tolist() == [0] and ri[0, :1].tolist() == [1]
    assert sh[1, :1].tolist() == [0] and le[1, :1].tolist() == [2] and ri[1, :1].tolist() == [3]
    assert (le[0] == -1).all() and (sh[0, 1:] == -1).all()


def test_pair_regions_closed_cases_and_partition():
    W = 9
    idx = np.full((5, W), -1, np.int32)
    vl = np.array([4, 4, 3, 2, 5], np.int32)
    idx[0, :4] = idx[1, :4] = [1, 5, 9, 12]          # identical rows
    idx[2, :3], idx[3, :2] = [0, 2, 4], [1, 3]       # disjoint rows; row 4 unpaired
    sh, le, ri, cnt = orc.pair_regions(idx, vl)
    assert cnt.tolist() == [[4, 0, 0], [0, 3, 2]]
    assert sh[0, :4].tolist() == [1, 5, 9, 12] and le[1, :3].tolist() == [0, 2, 4]
    rng = np.random.default_rng(5)
    for _ in range(200):
        a = np.unique(rng.integers(0, 60, size=rng.integers(0, 30)))
        b = np.unique(rng.integers(0, 60, size=rng.integers(0, 30)))
        idx = np.full((2, 64), -1, np.int32)
        idx[0, :a.size], idx[1, :b.size] = a, b
        sh, le, ri, cnt = orc.pair_regions(idx, np.array([a.size, b.size]))
        s_, l_, r_ = (set(x[0, :c].tolist()) for x, c in zip((sh, le, ri), cnt[0]))
        assert s_ | l_ == set(a.tolist()) and s_ | r_ == set(b.tolist())
        assert not (s_ & l_) and not (s_ & r_) and not (l_ & r_)
        for x, c in zip((sh, le, ri), cnt[0]):
            assert list(x[0, :c]) == sorted(x[0, :c]) and (x[0, c:] == -1).all()


def test_we2_tie_rule():
    rec = load("we2_tie_rule.txt")
    inp = _we_inputs(rec, S=5)
    got = orc.pair_scores(inp, [4] * 5, range(5))
    assert list(got) == [float(v) for v in rec["score"][0]]
    out = orc.select_rows(inp, [4])
    t, v, *ids = (int(x) for x in rec["row"][0])
    assert out["valid_len"][0] == v and list(out["idx"][0]) == ids
    # rank order: k3, k0, then the tie at 0 goes to the lower index k2
    assert list(out["key_idx"][0]) == [3, 0, 2]


@pytest.mark.parametrize("K", [1, 3, 8])
def test_all_zero_queries_every_key_ties(K):
    """q = 0 makes every score 0; the tie rule then picks the K lowest indices."""
    S = T = 20
    q = torch.zeros(S, 2, 3)
    k = torch.randn(T, 3, generator=torch.Generator().manual_seed(1))
    inp = gen.custom(q=q, k=k, w=torch.tensor([1.0, -1.0]), topk=K)
    out = orc.select_rows(inp, np.arange(S))
    for t in range(S):
        n = min(K, t + 1)
        assert list(out["idx"][t][:n]) == list(range(n))
        assert out["tau"][t] == 0.0


def test_we3_watch_lengths_and_width():
    rec = load("we3_watch_lengths.txt")
    m, topk, W = scalar(rec, "m"), scalar(rec, "topk"), scalar(rec, "width")
    assert orc.output_width(topk, m, True, True) == W
    assert orc.output_width(2048, 4, False, False) == 2048
    for L, pools, tl in (map(int, r) for r in rec["watch"]):
        p = L - 1
        assert orc.visible_keys(p, 10 ** 6, m, True) == pools
        assert orc.tail_len(p, 10 ** 6, m, True, True, True) == tl
    for p, v in (map(int, r) for r in rec["vlen"]):
        assert orc.expected_valid_len(p, 10 ** 6, m, topk, True, True, True) == v
    # the C oracle agrees at every watch length (tiny H, d; one pool-sized budget)
    S = 9
    T = S // m
    inp = gen.custom(q=torch.ones(S, 1, 1), k=torch.arange(1, T + 1, dtype=torch.float32)[:, None],
                     w=torch.ones(1), m=m, topk=8, expand=True, tail=True)
    out = orc.select_rows(inp, np.arange(S))
    for L, pools, tl in (map(int, r) for r in rec["watch"]):
        assert out["valid_len"][L - 1] == pools * m + tl
    # and the row of width 2051 is full at t = 2050 (topk 2048, m 4, 512 pools)
    S = 2051
    T = S // m
    inp = gen.custom(q=torch.ones(S, 1, 1), k=torch.ones(T, 1), w=torch.ones(1), m=m,
                     topk=topk, expand=True, tail=True)
    out = orc.select_rows(inp, [2046, 2047, 2050])
    assert list(out["valid_len"]) == [2047, 2048, 2051]
    assert list(out["idx"][2]) == list(range(2051))


def test_we4_pool_leak():
    rec = load("we4_pool_leak.txt")
    inp = _we_inputs(rec, S=9, expand=True, tail=True)
    out = orc.select_rows(inp, np.arange(9))
    for row in rec["row"]:
        t, v, *ids = (int(x) for x in row)
        assert out["valid_len"][t] == v, t
        assert list(out["idx"][t]) == ids, t
    # query 5 never sees positions 6 or 7, whatever the scores
    assert not ({6, 7} & set(out["idx"][5].tolist()))
    check_rows(out["idx"], out["valid_len"], range(9), T=2, m=4, topk=4, causal=True,
               expand=True, tail=True)


def _we6_inputs(rec, S, expand):
    k = torch.tensor([[float(v[0])] for v in rec["k"]])
    return gen.custom(q=torch.ones(S, 1, 1), k=k, w=torch.ones(1), m=scalar(rec, "m"),
                      topk=scalar(rec, "topk") if expand else 1, expand=expand, tail=expand)


def test_we6_packed_documents():
    rec = load("we6_packed_documents.txt")
    S = scalar(rec, "S")
    cu_q = [int(x) for x in rec["cu_q"][0]]
    cu_k = [int(x) for x in rec["cu_k"][0]]
    cu_tok = [int(x) for x in rec["cu_tok"][0]]
    out = orc.select_rows_varlen(_we6_inputs(rec, S, True), cu_q, cu_k, cu_tok=cu_tok)
    for row in rec["exp"]:
        t, v, *ids = (int(x) for x in row)
        assert out["valid_len"][t] == v, t
        assert list(out["idx"][t]) == ids, t
    out = orc.select_rows_varlen(_we6_inputs(rec, S, False), cu_q, cu_k)
    for row in rec["cmp"]:
        t, v, *ids = (int(x) for x in row)
        assert out["valid_len"][t] == v, t
        assert list(out["idx"][t]) == ids, t
    dq = [int(x) for x in rec["dec_cu_q"][0]]
    dp = [int(x) for x in rec["dec_pos0"][0]]
    out = orc.select_rows_varlen(_we6_inputs(rec, 10, True), dq, cu_k, pos0=dp, cu_tok=cu_tok)
    for row in rec["dec"]:
        t, v, *ids = (int(x) for x in row)
        assert out["valid_len"][t] == v, t
        assert list(out["idx"][t]) == ids, t


def test_varlen_matches_brute_force_per_document():
    """Random packed batches of tiny integer documents (lengths around the
    pool edges, padding rows, later-chunk positions): every row equals the
    brute-force selection over its own document's keys, offset to global
    indices, and no row ever names another document's key or token."""
    rng = np.random.default_rng(20261204)
    for case in range(300):
        m = int(rng.choice([1, 2, 4]))
        H, d = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        expand = bool(m > 1 and rng.random() < 0.5)
        topk = int(rng.integers(1, 5)) * (m if expand else 1)
        ndoc = int(rng.integers(1, 5))
        lens = rng.choice([1, 2, 3, 4, 5, 7, 8, 9, 12], size=ndoc)
        pos0 = rng.integers(0, 6, size=ndoc)
        nkeys = [(int(p) + int(n)) // m for p, n in zip(pos0, lens)]  # every complete pool
        cu_q = np.concatenate([[0], np.cumsum(lens)])
        cu_k = np.concatenate([[0], np.cumsum(nkeys)])
        cu_tok = np.concatenate([[0], np.cumsum([int(p) + int(n) for p, n in zip(pos0, lens)])])[:-1]
        S, T = int(cu_q[-1]) + int(rng.integers(0, 3)), int(cu_k[-1])
        q = torch.from_numpy(rng.integers(-3, 4, size=(S, H, d)).astype(np.float32))
        k = torch.from_numpy(rng.integers(-3, 4, size=(max(T, 1), d)).astype(np.float32))[:T]
        w = torch.from_numpy(rng.choice([-1.0, -0.5, 0.5, 1.0], size=H).astype(np.float32))
        inp = gen.custom(q=q, k=k, w=w, m=m, topk=topk, expand=expand, tail=expand)
        out = orc.select_rows_varlen(inp, cu_q, cu_k, pos0=pos0, cu_tok=cu_tok)
        Q, Wt, K = dequant(inp)
        for t in range(S):
            i = int(np.searchsorted(cu_q, t, side="right")) - 1
            if i >= ndoc:
                assert out["valid_len"][t] == 0 and np.all(out["idx"][t] == -1), (case, t)
                continue
            p = int(pos0[i]) + t - int(cu_q[i])
            Kd = K[cu_k[i]:cu_k[i + 1]]
            pos, _, _ = brute_row(Q[t], Wt[t], Kd, p, Kd.shape[0], m, topk, True, expand, expand)
            want = pos + (cu_tok[i] if expand else cu_k[i])
            v = len(want)
            assert out["valid_len"][t] == v, (case, t)
            assert list(out["idx"][t][:v]) == list(want), (case, t)
            lo, hi = (cu_tok[i], cu_tok[i] + int(pos0[i]) + lens[i]) if expand else \
                (cu_k[i], cu_k[i + 1])
            assert all(lo <= x < hi for x in out["idx"][t][:v]), (case, t)


def test_we5_csa_counts():
    rec = load("we5_csa_counts.txt")
    m, topk = scalar(rec, "m"), scalar(rec, "topk")
    for p, v in (map(int, r) for r in rec["vlen"]):
        assert orc.expected_valid_len(p, 10 ** 6, m, topk, True, False, False) == v
    T = 8192
    inp = gen.custom(q=torch.ones(8192, 1, 1), k=torch.ones(T, 1), w=torch.ones(1), m=m,
                     topk=topk)
    rows = [int(r[0]) for r in rec["vlen"] if int(r[0]) < 8192]
    out = orc.select_rows(inp, rows)
    for r, t in enumerate(rows):
        v = orc.expected_valid_len(t, T, m, topk, True, False, False)
        assert out["valid_len"][r] == v
    assert list(out["idx"][rows.index(3)][:2]) == [0, -1]


def test_tail_needs_every_complete_pool():
    """With the tail on, T must cover every complete pool, else the tail would
    exceed m-1 positions; the oracle refuses such a problem."""
    inp = gen.custom(q=torch.ones(12, 1, 1), k=torch.ones(2, 1), w=torch.ones(1), m=4, topk=4,
                     expand=True, tail=True)
    with pytest.raises(RuntimeError):
        orc.select_rows(inp, [11])


def _random_tiny(rng):
    S = int(rng.integers(1, 17))
    m = int(rng.integers(1, 5))
    expand = bool(rng.integers(0, 2)) and m > 1
    tail = expand and bool(rng.integers(0, 2))
    causal = bool(rng.integers(0, 4) > 0)
    q_pos0 = int(rng.integers(0, 5)) if causal else 0
    T = int(rng.integers(1, 17)) if not tail else max(1, (S + q_pos0) // m + int(rng.integers(0, 3)))
    H = int(rng.integers(1, 4))
    d = int(rng.integers(1, 5))
    units = T * (m if expand else 1)
    topk = int(rng.integers(1, units + 2))
    if expand:
        topk = max(m, (topk // m) * m)
    q = torch.from_numpy(rng.integers(-3, 4, (S, H, d)).astype(np.float32))
    k = torch.from_numpy(rng.integers(-3, 4, (T, d)).astype(np.float32))
    wv = np.array([-2, -1, -0.5, 0.5, 1, 2], np.float32)
    if rng.integers(0, 2):
        w = torch.from_numpy(wv[rng.integers(0, 6, (S, H))])
    else:
        w = torch.from_numpy(wv[rng.integers(0, 6, (H,))])
    inp = gen.custom(q=q, k=k, w=w, m=m, topk=topk, causal=causal, expand=expand, tail=tail,
                     q_pos0=q_pos0)
    return inp


def test_oracle_matches_brute_force_on_random_tiny_cases():
    """Integer inputs make every score exact in fp64, so rows must match
    exactly, ties included (they are frequent with values in [-3, 3])."""
    rng = np.random.default_rng(20261203)
    for case in range(4000):
        inp = _random_tiny(rng)
        out = orc.select_rows(inp, np.arange(inp.S))
        Q, Wt, K = dequant(inp)
        for t in range(inp.S):
            p = t + inp.q_pos0
            pos, sel, s = brute_row(Q[t], Wt[t], K, p, inp.T, inp.m, inp.topk, inp.causal,
                                    inp.expand, inp.tail)
            v = len(pos)
            assert out["valid_len"][t] == v, (case, t)
            assert list(out["idx"][t][:v]) == list(pos), (case, t)
            assert np.all(out["idx"][t][v:] == -1)
            n = out["n_sel"][t]
            assert set(out["key_idx"][t][:n].tolist()) == sel, (case, t)
            np.testing.assert_array_equal(out["key_score"][t][:n], s[out["key_idx"][t][:n]])


def test_reduces_to_stable_argsort():
    """H = 1, w = +1, q and k positive: s = q . k, so the selection is the
    first K entries of a stable descending argsort (lower index first on ties)."""
    g = torch.Generator().manual_seed(7)
    S, T, d, K = 6, 300, 16, 37
    q = torch.rand(S, 1, d, generator=g) + 0.01
    k = torch.rand(T, d, generator=g) + 0.01
    inp = gen.custom(q=q, k=k, w=torch.ones(1), topk=K, causal=False)
    out = orc.select_rows(inp, np.arange(S))
    for t in range(S):
        s = k.double().numpy() @ q[t, 0].double().numpy()
        want = np.argsort(-s, kind="stable")[:K]
        assert list(out["key_idx"][t]) == list(want)
        assert list(out["idx"][t]) == sorted(want)


def test_decode_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().double().numpy()
    for c in range(256):
        got = orc.decode_e4m3(c)
        if np.isnan(ref[c]):
            assert np.isnan(got), c
        else:
            assert got == ref[c], c
    assert orc.decode_e4m3(0x7E) == 448.0 and orc.decode_e4m3(0x01) == 2.0 ** -9


def test_decode_bf16_all_codes_match_torch():
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = codes.view(torch.bfloat16).float().double().numpy()
    got = np.array([orc.decode_bf16(c) for c in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


@pytest.mark.parametrize("name", ["c2_glm_pooled", "c3_dsa_token", "c5_csa_1m"])
def test_scaled_configs_match_brute_force(name):
    """bf16 and fp8-with-scales inputs: the oracle's hand decoders and scale
    handling against torch's casts; float scores, so compare selections by
    score (ties are measure-zero here) and the scores to fp64 rounding."""
    inp = gen.generate(name, S=96, topk=16 if name != "c2_glm_pooled" else 32)
    inp.q_pos0 = 0
    out = orc.select_rows(inp, np.arange(inp.S))
    Q, Wt, K = dequant(inp)
    for t in range(inp.S):
        pos, sel, s = brute_row(Q[t], Wt[t], K, t, inp.T, inp.m, inp.topk, inp.causal,
                                inp.expand, inp.tail)
        v = len(pos)
        assert out["valid_len"][t] == v
        assert list(out["idx"][t][:v]) == list(pos)
        n = out["n_sel"][t]
        np.testing.assert_allclose(out["key_score"][t][:n], s[out["key_idx"][t][:n]],
                                   rtol=1e-12, atol=1e-14)
    check_rows(out["idx"], out["valid_len"], range(inp.S), T=inp.T, m=inp.m, topk=inp.topk,
               causal=inp.causal, expand=inp.expand, tail=inp.tail)


def test_page1_overlap_numbers_pin_the_denominator():
    """Page-1 means satisfy overlap = shared / min(vA, vB) with causal-prefix
    pairs A = {0..2i} c B = {0..2i+1}, and full rows of 2048 afterwards; a
    fixed 2048 denominator misses step 0 by ~0.4 pp."""
    rec = load("page1_overlap_table.txt")
    S, K = 262144, 2048
    npairs = S // 2
    npre = K // 2
    i = np.arange(npairs)
    va = np.where(i < npre, 2 * i + 1, K)
    vb = np.where(i < npre, 2 * i + 2, K)
    vl = np.empty(S, np.int64)
    vl[0::2], vl[1::2] = va, vb
    for step, ov_pct, mean_shared in ((int(a), float(b), float(c)) for a, b, c in rec["step"]):
        total = int(round(mean_shared * npairs)) - npre * npre
        rest = npairs - npre
        base, extra = divmod(total, rest)
        sh = np.where(i < npre, 2 * i + 1, base)
        sh[npre:npre + extra] += 1
        st = orc.overlap_stats(sh, vl)
        assert st["mean_shared"] == pytest.approx(mean_shared, abs=0.05)
        assert abs(st["mean_overlap"] * 100 - ov_pct) < 0.01, (step, st["mean_overlap"])
        fixed = sh.sum() / K / npairs
        if step == 0:
            assert abs(fixed * 100 - ov_pct) > 0.3


def test_pair_overlap_closed_cases():
    rng = np.random.default_rng(3)
    W = 50
    rows = []
    for _ in range(40):
        v = int(rng.integers(0, W + 1))
        rows.append(np.sort(rng.choice(200, v, replace=False)))
    idx = -np.ones((40, W), np.int32)
    vl = np.zeros(40, np.int32)
    for r, a in enumerate(rows):
        idx[r, :len(a)], vl[r] = a, len(a)
    sh = orc.pair_overlap(idx, vl)
    for p in range(20):
        assert sh[p] == len(set(rows[2 * p]) & set(rows[2 * p + 1]))
    same = np.repeat(idx[:1], 2, 0)
    assert orc.pair_overlap(same, np.repeat(vl[:1], 2))[0] == vl[0]
    dis = np.array([[0, 2, 4], [1, 3, 5]], np.int32)
    assert orc.pair_overlap(dis, np.array([3, 3]))[0] == 0
    # an odd last row has no partner
    assert orc.pair_overlap(idx[:5], vl[:5]).shape == (2,)


def test_invariant_checker_catches_planted_mistakes():
    """The row checker used by the GPU parity tests rejects the mistakes it
    is meant to catch (mistakes planted into oracle output, on the CPU)."""
    inp = gen.generate("c2_glm_pooled", S=64, topk=16)
    out = orc.select_rows(inp, np.arange(64))
    kw = dict(T=inp.T, m=4, topk=16, causal=True, expand=True, tail=True)
    check_rows(out["idx"], out["valid_len"], range(64), **kw)
    bad = out["idx"].copy()
    bad[40, 0], bad[40, 1] = bad[40, 1], bad[40, 0]            # order
    with pytest.raises(AssertionError):
        check_rows(bad, out["valid_len"], range(64), **kw)
    bad = out["idx"].copy()
    v = out["valid_len"][5]
    bad[5, v - 1] = 7                                           # a future position
    with pytest.raises(AssertionError):
        check_rows(bad, out["valid_len"], range(64), **kw)
    badv = out["valid_len"].copy()
    badv[63] -= 1                                               # wrong length
    with pytest.raises(AssertionError):
        check_rows(out["idx"], badv, range(64), **kw)


def test_pair_bounds_closed_forms():
    """B = sum_h |w_h| sum_i |q_hi k_i|: hand value on WE1, equal to the score
    when every term is non-negative, and never below |s| (triangle inequality)."""
    rec = load("we1_signed_relu.txt")
    inp = _we_inputs(rec, S=4)
    b = orc.pair_scores(inp, [3] * 4, [0, 1, 2, 3], bounds=True)
    assert list(b) == [3.0, 4.0, 2.0, 5.0]   # k0=(2,1): 2+1, k1: 1+3, k2: 1+1, k3: 3+2
    g = torch.Generator().manual_seed(9)
    pos = gen.custom(q=torch.rand(8, 3, 16, generator=g), k=torch.rand(40, 16, generator=g),
                     w=torch.rand(3, generator=g), topk=4, causal=False)
    rows, keys = np.repeat(np.arange(8), 40), np.tile(np.arange(40), 8)
    np.testing.assert_allclose(orc.pair_scores(pos, rows, keys, bounds=True),
                               orc.pair_scores(pos, rows, keys), rtol=1e-14)
    mix = gen.generate("c3_dsa_token", S=32, topk=8)
    rows, keys = np.repeat(np.arange(32), 32), np.tile(np.arange(32), 32)
    s = orc.pair_scores(mix, rows, keys)
    bb = orc.pair_scores(mix, rows, keys, bounds=True)
    assert np.all(bb >= np.abs(s)) and np.any(bb > 1.5 * np.abs(s))
