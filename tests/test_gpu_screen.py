"""DoSA certificate screening (IDX_SCREEN) on the GPU.

"DoSA: Dots Sparse Attention" (summary page, "Core method", "Method
steps"): certificates are checked against the oracle's construction
(oracle/dosa.py, empty seed set) and against their defining inequality
U >= s on every key; the screened selection is lossless, so it passes the
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


def _cert_rows(inp, rows):
    import dsa_indexer_score_amd as dsai
    perm, wv, wt, e = dsai.screen_certificates(inp.q, inp.w, inp.q_scale)
    torch.cuda.synchronize()
    return perm.cpu().numpy()[rows], wv.cpu().numpy()[rows], wt.cpu().numpy()[rows], \
        e.cpu().numpy()[rows]


def _check_certificates(inp, rows, keys_real, kscale):
    """GPU certificates of the given rows against the oracle's and against
    U >= s on every key (fp64 evaluation of the GPU's numbers)."""
    perm, wv, wt, e = _cert_rows(inp, rows)
    q = _real(inp.q)
    qs = np.ones((inp.S, inp.H)) if inp.q_scale is None else _real(inp.q_scale)
    w = _real(inp.w)
    w = np.broadcast_to(w, (inp.S, inp.H)) if w.ndim == 1 else w
    folds = 0
    for n, t in enumerate(rows):
        H = inp.H
        assert sorted(perm[n][perm[n] >= 0].tolist()) == list(range(H))
        a = w[t] * qs[t]
        np.testing.assert_allclose(wv[n][:H], a[perm[n][:H]], rtol=1e-6)
        qreal = q[t] * qs[t][:, None]
        cert = dosa.certificate(qreal, w[t], np.zeros((0, inp.d)), r=32)
        kept = perm[n][:32]
        assert sorted(kept.tolist()) == sorted(cert["kept"]), t
        fold_of = dict(zip(cert["kept"], cert["w_fold"]))
        want_wt = np.array([qs[t][j] * fold_of[j] for j in kept])
        np.testing.assert_allclose(wt[n], want_wt, rtol=2e-5, atol=1e-6 * np.abs(a).max())
        C = np.sum(np.abs(a) * np.linalg.norm(q[t], axis=1))
        assert cert["E"] * (1 - 1e-5) <= e[n] <= cert["E"] * (1 + 1e-4) + 1e-3 * C, t
        folds += cert["E"] > 0
        # the bound, evaluated in fp64 from the GPU's numbers, covers every key
        s = a @ np.maximum(q[t] @ keys_real.T, 0.0)
        U = wt[n] @ np.maximum(q[t][kept] @ keys_real.T, 0.0) + \
            e[n] * np.linalg.norm(keys_real, axis=1)
        assert np.all(U * kscale >= s * kscale - 1e-12), t
    return folds


@pytest.mark.parametrize("name", ["c4_csa_256k", "c5_csa_1m", "c3_dsa_token"])
def test_certificates_match_oracle(name):
    inp = gen.generate(name, S=64, T=2048).to(DEV)
    rows = np.arange(0, 64, 3)
    k = _real(inp.k)
    ks = np.ones(inp.T) if inp.k_scale is None else _real(inp.k_scale)
    folds = _check_certificates(inp, rows, k, ks)
    log(f"  {name}: {rows.size} rows, {folds} with folded positive heads")


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
    folds = _check_certificates(inp, rows, k, ks)
    assert folds == rows.size


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


def test_screened_full_size_sampled_rows():
    """The 256K workload at full size in its benchmark launch configuration
    (16 query chunks), screened: sampled rows against the oracle's rule,
    every row against the device invariants."""
    from gpu_util import device_invariants, rows_to_host
    inp = gen.generate("c4_csa_256k", device=DEV)
    idx, vl, sc = run(inp, screen=True)
    device_invariants(inp, idx, vl)
    rows = check.sample_rows(inp.S, m=inp.m, ksel=inp.topk, chunk=inp.query_chunk,
                             seed=inp.seed, n_uniform=96)
    hi, hv, hs = rows_to_host(rows, idx, vl, sc)
    rep = check.compare(inp, rows, hi, hv, hs)
    log(f"  rows {rep['rows']}, index-mismatch rows {rep['index_mismatch_rows']}")
    assert rep["ok"], rep["failures"][:3]
