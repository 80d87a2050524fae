"""DoSA certificate screening (IDX_SCREEN) on the GPU.

"DoSA: Dots Sparse Attention" (summary page, "Core method", "Method
steps"): certificates are checked against the oracle's construction
(oracle/dosa.py, with the seed activation counts the GPU measured, or
an empty seed set) and against their defining inequality U >= s on every
key; the screened selection is lossless, so it passes the
oracle's tolerance rule, and on integer-valued inputs (every sum exact in
any order) it equals the unscreened selection bit for bit.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from gpu_util import log, run
from oracle import check, dosa
from workloads import gen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _real(t):
    return t.float().double().cpu().numpy()


def _cert_rows(inp, rows, seeds):
    import dsa_indexer_score_amd as dsai
    out = dsai.screen_certificates(inp.q, inp.w, inp.q_scale, inp.k if seeds else None,
                                   m=inp.m, causal=inp.causal, q_pos0=inp.q_pos0)
    torch.cuda.synchronize()
    return [x.cpu().numpy()[rows] for x in out]


def _seed_positions(inp, t):
    """The seed set the certificate uses: n_s = min(P, 256) of the row's P
    visible keys, key i P // n_s for i < n_s."""
    P = min((inp.q_pos0 + t + 1) // inp.m, inp.T) if inp.causal else inp.T
    ns = min(P, 256)
    return (np.arange(ns, dtype=np.int64) * P) // max(ns, 1)


def _check_certificates(inp, rows, keys_real, kscale, seeds=True):
    """GPU certificates of the given rows against the oracle's and against
    U >= s on every key (fp64 evaluation of the GPU's numbers).  Seed
    activation counts must equal the fp64 counts except for dot products
    within rounding of zero; the oracle then takes the GPU's counts, so the
    rest of the construction is compared on equal footing."""
    perm, wv, wt, e, agg, act = _cert_rows(inp, rows, seeds)
    q = _real(inp.q)
    qs = np.ones((inp.S, inp.H)) if inp.q_scale is None else _real(inp.q_scale)
    w = _real(inp.w)
    w = np.broadcast_to(w, (inp.S, inp.H)) if w.ndim == 1 else w
    stats = dict(folds=0, aggregates=0, agg_heads=0)
    H = inp.H
    for n, t in enumerate(rows):
        a = w[t] * qs[t]
        qreal = q[t] * qs[t][:, None]
        C = np.sum(np.abs(a) * np.linalg.norm(q[t], axis=1))
        sp = _seed_positions(inp, t) if seeds else np.zeros(0, np.int64)
        ns = sp.size
        X = q[t] @ keys_real[sp].T                       # codes: signs ignore the scales
        cnt = (X > 0).sum(axis=1)
        near = (np.abs(X) <= 1e-5 * np.linalg.norm(q[t], axis=1)[:, None]
                * np.linalg.norm(keys_real[sp], axis=1)[None, :]).sum(axis=1)
        assert np.all(np.abs(act[n][:H] - cnt) <= near), (t, act[n][:H] - cnt)
        assert np.all(act[n][H:] == 0)
        has_agg = ns > 0 and H <= 63
        r = 31 if has_agg else 32
        cert = dosa.certificate(qreal, w[t], keys_real[sp], r=r,
                                p=act[n][:H] / ns if ns else None)
        heads = perm[n][perm[n] >= 0]
        assert sorted(heads.tolist()) == list(range(H)), t
        kept = perm[n][:r]
        assert sorted(kept.tolist()) == sorted(cert["kept"]), t
        assert list(kept) == sorted(kept), t                # by head index
        assert (perm[n][31] == -2) == has_agg, t
        np.testing.assert_allclose(wv[n][perm[n] >= 0], a[heads], rtol=1e-6)
        fold_of = dict(zip(cert["kept"], cert["w_fold"]))
        want_wt = np.array([qs[t][j] * fold_of[j] for j in kept])
        np.testing.assert_allclose(wt[n][:r], want_wt, rtol=2e-5, atol=1e-6 * np.abs(a).max())
        aA = cert["aA"]
        if has_agg:
            assert wt[n][31] == -1.0 and wv[n][31] == 0.0, t
            # a_A rounded to bf16 (fp32 data: fp32 rounding of the sum)
            rel = 2.0 ** -8 if inp.q.dtype != torch.float32 else 1e-6
            np.testing.assert_allclose(agg[n], aA, rtol=rel, atol=1e-5 * C)
            stats["aggregates"] += 1
            stats["agg_heads"] += len(cert["A"])
        lo = min(cert["E"], cert["E_joint"])
        slack = 2.0 ** -8 * np.linalg.norm(aA) + 1e-3 * C
        assert lo * (1 - 1e-4) - 1e-6 * C <= e[n] <= lo * (1 + 1e-4) + slack, t
        stats["folds"] += cert["E"] > 0
        # the bound, evaluated in fp64 from the GPU's numbers, covers every key
        s = a @ np.maximum(q[t] @ keys_real.T, 0.0)
        kh = perm[n][:32]
        U = wt[n][:r] @ np.maximum(q[t][kh[:r]] @ keys_real.T, 0.0) + \
            e[n] * np.linalg.norm(keys_real, axis=1)
        if has_agg:
            U -= np.maximum(keys_real @ agg[n], 0.0)
        assert np.all(U * kscale >= s * kscale - 1e-12), t
    return stats


@pytest.mark.parametrize("name", ["c4_csa_256k", "c5_csa_1m", "c3_dsa_token"])
def test_certificates_match_oracle(name):
    inp = gen.generate(name, S=64, T=2048).to(DEV)
    rows = np.arange(0, 64, 3)
    k = _real(inp.k)
    ks = np.ones(inp.T) if inp.k_scale is None else _real(inp.k_scale)
    st = _check_certificates(inp, rows, k, ks)
    log(f"  {name}: {rows.size} rows, {st}")
    st0 = _check_certificates(inp, rows, k, ks, seeds=False)
    assert st0["aggregates"] == 0


def _many_positive(S, H, d, T, dtype, shared, seed):
    """Rows with more than 32 positive heads (forces folding) whose heads
    share one direction, so the bound is tight and prunes."""
    g = torch.Generator().manual_seed(seed)
    base = torch.randn(S, 1, d, generator=g)
    q = (shared * base + (1 - shared ** 2) ** 0.5 * torch.randn(S, H, d, generator=g)) / d ** 0.5
    k = torch.randn(T, d, generator=g) / d ** 0.5
    w = torch.randn(S, H, generator=g).abs()
    w[:, 40:] = -w[:, 40:]                              # 40 positive heads, H - 40 negative
    fp8 = dtype == torch.float8_e4m3fn
    if fp8:
        qs = q.abs().amax(-1) / 448 + 1e-12
        ks = k.abs().amax(-1) / 448 + 1e-12
        q, k = (q / qs[..., None]).to(dtype), (k / ks[:, None]).to(dtype)
    else:
        q, k, qs, ks = q.to(dtype), k.to(dtype), None, None
    return gen.custom(q=q, k=k, w=w, topk=64, q_scale=qs, k_scale=ks)


@pytest.mark.parametrize("dtype,H,d", [(torch.bfloat16, 64, 128), (torch.float8_e4m3fn, 48, 64),
                                       (torch.float32, 40, 32)])
def test_certificates_fold_positive_heads(dtype, H, d):
    inp = _many_positive(24, H, d, 700, dtype, 0.9, H + d).to(DEV)
    rows = np.arange(24)
    k = _real(inp.k)
    ks = np.ones(inp.T) if inp.k_scale is None else _real(inp.k_scale)
    st = _check_certificates(inp, rows, k, ks)
    assert st["folds"] == rows.size
    assert st["aggregates"] == (rows.size if H <= 63 else 0)
    log(f"  {dtype} H={H} d={d}: {st}")


def _skewed(S, H, d, T, dtype, seed):
    """Heads whose activation frequencies sit far from 1/2: keys share a
    direction u, each head leans towards +u or -u; weights are signed at
    random (about half negative), so majority-active negative heads exist
    and the seed statistics decide which negative heads are kept."""
    g = torch.Generator().manual_seed(seed)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    lean = torch.where(torch.rand(S, H, generator=g) < 0.5, -1.0, 1.0)
    q = (torch.randn(S, H, d, generator=g) / d ** 0.5 + 1.5 * lean[..., None] * u) / 2
    k = torch.randn(T, d, generator=g) / d ** 0.5 + u
    w = torch.randn(S, H, generator=g)
    fp8 = dtype == torch.float8_e4m3fn
    if fp8:
        qs = q.abs().amax(-1) / 448 + 1e-12
        ks = k.abs().amax(-1) / 448 + 1e-12
        q, k = (q / qs[..., None]).to(dtype), (k / ks[:, None]).to(dtype)
    else:
        q, k, qs, ks = q.to(dtype), k.to(dtype), None, None
    return gen.custom(q=q, k=k, w=w, topk=64, q_scale=qs, k_scale=ks)


@pytest.mark.parametrize("dtype,H,d", [(torch.bfloat16, 48, 128), (torch.bfloat16, 63, 64),
                                       (torch.float8_e4m3fn, 56, 128),
                                       (torch.float32, 40, 64), (torch.bfloat16, 64, 128)])
def test_certificates_with_seed_statistics(dtype, H, d):
    """Skewed activation frequencies: the seed counts, the negative heads
    kept by |a_h| ||q_h|| min(p_h, 1 - p_h), the aggregate of the
    majority-active omitted negative heads (H <= 63) and U >= s on every
    key, against the oracle."""
    inp = _skewed(20, H, d, 900, dtype, 5 * H + d).to(DEV)
    rows = np.arange(20)
    k = _real(inp.k)
    ks = np.ones(inp.T) if inp.k_scale is None else _real(inp.k_scale)
    st = _check_certificates(inp, rows, k, ks)
    log(f"  {dtype} H={H} d={d}: {st}")
    if H <= 63:
        assert st["aggregates"] == rows.size and st["agg_heads"] >= rows.size


@pytest.mark.parametrize("dtype,H,d", [(torch.bfloat16, 48, 128), (torch.float8_e4m3fn, 56, 64),
                                       (torch.float32, 40, 32)])
def test_screened_selection_with_aggregate(dtype, H, d):
    """Screened selection with the aggregate row in use (skewed activation
    frequencies, H <= 63): lossless against the oracle's rule."""
    inp = _skewed(1200, H, d, 1200, dtype, 7 * H + d).to(DEV)
    idx, vl, sc = run(inp, screen=True)
    rows = np.arange(0, 1200, 5)
    rep = check.compare(inp, rows, idx.cpu().numpy()[rows], vl.cpu().numpy()[rows],
                        sc.cpu().numpy()[rows])
    assert rep["ok"], rep["failures"][:3]


@pytest.mark.parametrize("name,S", [("c4_csa_256k", 3000), ("c3_dsa_token", 2500),
                                    ("c5_csa_1m", 3000)])
def test_screened_selection_matches_oracle(name, S):
    inp = gen.generate(name, S=S, topk=512 if name != "c3_dsa_token" else 256).to(DEV)
    idx, vl, sc = run(inp, screen=True)
    rows = check.sample_rows(S, m=inp.m, ksel=inp.topk // inp.m if inp.expand else inp.topk,
                             n_uniform=64)
    rep = check.compare(inp, rows, idx.cpu().numpy()[rows], vl.cpu().numpy()[rows],
                        sc.cpu().numpy()[rows])
    assert rep["ok"], rep["failures"][:3]
    base = run(inp)
    assert torch.equal(base[1], vl)
    same = (base[0] == idx).all(dim=1).float().mean().item()
    log(f"  {name} S={S}: screened rows identical to unscreened: {same:.4f}")


@pytest.mark.parametrize("shared", [0.0, 0.9])
def test_screened_integer_inputs_equal_unscreened_bit_for_bit(shared):
    """fp32 holding small integers, H = 48 with 40 positive heads: every
    score is exact whatever the summation order, so the screened selection
    equals the unscreened one exactly; the oracle agrees bit for bit."""
    g = torch.Generator().manual_seed(7 + int(shared * 10))
    S, T, H, d = 700, 700, 48, 32
    base = torch.randint(-3, 4, (S, 1, d), generator=g).float()
    noise = torch.randint(-1, 2, (S, H, d), generator=g).float()
    q = base + noise if shared else torch.randint(-3, 4, (S, H, d), generator=g).float()
    k = torch.randint(-3, 4, (T, d), generator=g).float()
    w = torch.tensor([1.0, 0.5] * 20 + [-1.0, -0.5] * 4).repeat(S, 1)
    inp = replace(gen.custom(q=q, k=k, w=w, topk=48), meta={"qdist": "int"}).to(DEV)
    plain = run(inp)
    scr = run(inp, screen=True)
    for a, b in zip(plain, scr):
        assert torch.equal(a, b)
    rep = check.compare(inp, np.arange(0, S, 7), scr[0].cpu().numpy()[::7],
                        scr[1].cpu().numpy()[::7], exact=True)
    assert rep["ok"], rep["failures"][:3]


@pytest.mark.parametrize("dtype,H,d", [(torch.bfloat16, 64, 128), (torch.float8_e4m3fn, 48, 64),
                                       (torch.float32, 40, 32)])
def test_screened_selection_with_folds_and_pruning(dtype, H, d):
    inp = _many_positive(1500, H, d, 1500, dtype, 0.9, 3 * H + d).to(DEV)
    idx, vl, sc = run(inp, screen=True)
    rows = np.arange(0, 1500, 5)
    rep = check.compare(inp, rows, idx.cpu().numpy()[rows], vl.cpu().numpy()[rows],
                        sc.cpu().numpy()[rows])
    assert rep["ok"], rep["failures"][:3]


def test_screened_selection_on_dominant_heads():
    """Head weights spread over decades (the stand-in where the certificate
    prunes): the screened selection still passes the oracle's rule."""
    inp = gen.generate("c4_csa_256k", S=3000, topk=512, wdist="lognormal_bcast").to(DEV)
    idx, vl, sc = run(inp, screen=True)
    rows = check.sample_rows(3000, m=inp.m, ksel=inp.topk, n_uniform=64)
    rep = check.compare(inp, rows, idx.cpu().numpy()[rows], vl.cpu().numpy()[rows],
                        sc.cpu().numpy()[rows])
    assert rep["ok"], rep["failures"][:3]


def test_screened_chunked_launches_and_modes():
    """Certificates are built per launch: several query chunks give the same
    result as one launch, bit for bit; expansion with the tail, a query
    offset and the non-causal mode pass the oracle's rule screened."""
    inp = gen.generate("c4_csa_256k", S=2500, topk=512).to(DEV)
    one = run(inp, screen=True, query_chunk=0)
    many = run(inp, screen=True, query_chunk=384)
    for a, b in zip(one, many):
        assert torch.equal(a, b)
    g = torch.Generator().manual_seed(31)
    S, H, d, m = 900, 48, 64, 4
    T = (37 + S) // m
    q = (torch.randn(S, H, d, generator=g) / d ** 0.5).bfloat16()
    k = (torch.randn(T, d, generator=g) / d ** 0.5).bfloat16()
    w = torch.randn(H, generator=g)
    for causal, expand, tail in ((True, True, True), (False, False, False)):
        inp = gen.custom(q=q, k=k, w=w, m=m, topk=256, causal=causal, expand=expand,
                         tail=tail, q_pos0=37 if causal else 0).to(DEV)
        idx, vl, sc = run(inp, screen=True, query_chunk=256)
        rows = np.arange(0, S, 4)
        rep = check.compare(inp, rows, idx.cpu().numpy()[rows], vl.cpu().numpy()[rows],
                            sc.cpu().numpy()[rows])
        assert rep["ok"], (causal, rep["failures"][:3])


@pytest.mark.parametrize("name", ["c4_csa_256k", "c3_dsa_token"])
def test_screened_full_size_sampled_rows(name):
    """The 256K-query (bf16) and 128K-token (fp8) workloads at full size in
    their benchmark launch configurations, screened: sampled rows against
    the oracle's rule, every row against the device invariants."""
    from gpu_util import device_invariants, rows_to_host
    inp = gen.generate(name, device=DEV)
    idx, vl, sc = run(inp, screen=True)
    device_invariants(inp, idx, vl)
    rows = check.sample_rows(inp.S, m=inp.m, ksel=inp.topk, chunk=inp.query_chunk,
                             seed=inp.seed, n_uniform=96)
    hi, hv, hs = rows_to_host(rows, idx, vl, sc)
    rep = check.compare(inp, rows, hi, hv, hs)
    log(f"  rows {rep['rows']}, index-mismatch rows {rep['index_mismatch_rows']}")
    assert rep["ok"], rep["failures"][:3]


@pytest.mark.parametrize("name,S,heads", [("c4_csa_256k", 2500, None), ("c4_csa_256k", 2500, 48)])
def test_screening_statistics(name, S, heads):
    """The call's statistics in the workspace's first 16 bytes: every
    visible key of every row is tested once, and every key of the final
    selection (at least the first Ksel of each row) passes."""
    import dsa_indexer_score_amd as dsai
    over = {} if heads is None else {"H": heads}
    inp = gen.generate(name, S=S, topk=512, **over).to(DEV)
    ix = dsai.Indexer(inp.q.dtype, expand=inp.expand, tail=inp.tail, query_chunk=1024,
                      few_query_rows=-1, screen=True, device=DEV)
    ws = torch.empty(ix.workspace_bytes(inp.S, inp.T, inp.H, inp.d, inp.m, inp.topk),
                     dtype=torch.uint8, device=DEV)
    kw = dict(m=inp.m, topk=inp.topk, causal=inp.causal, q_scale=inp.q_scale,
              k_scale=inp.k_scale, q_pos0=inp.q_pos0, with_scores=True, workspace=ws)
    out = ix.score_topk(inp.q, inp.w, inp.k, **kw)
    torch.cuda.synchronize()
    tested, passed = ws[:16].view(torch.int64).cpu().tolist()
    pos = np.arange(inp.S) + inp.q_pos0
    P = np.minimum((pos + 1) // inp.m, inp.T)
    ksel = inp.topk // inp.m if inp.expand else inp.topk
    assert tested == int(P.sum())
    assert int(np.minimum(P, ksel).sum()) <= passed <= tested
    log(f"  {name} H={inp.H}: {passed}/{tested} keys passed the bound ({passed / tested:.3f})")
    # a second call starts from zero
    ix.score_topk(inp.q, inp.w, inp.k, **kw)
    torch.cuda.synchronize()
    assert ws[:16].view(torch.int64).cpu().tolist() == [tested, passed]
    rows = np.arange(0, S, 11)
    rep = check.compare(inp, rows, out[0].cpu().numpy()[rows], out[1].cpu().numpy()[rows],
                        out[2].cpu().numpy()[rows])
    assert rep["ok"], rep["failures"][:3]
