"""The DoSA certificate (oracle/dosa.py) against what the page's inequalities
fix, and its survival rate on the synthetic workload.

"DoSA: Dots Sparse Attention" (summary page, "Core method", "Method
steps"): lossless screening needs U_i >= s_i for every key; with every head
kept the certificate is the score itself; a head that is a positive
multiple of a kept head folds into it exactly.
"""
import numpy as np
import pytest

from oracle import dosa
from workloads import gen


def _scores(q, w, keys):
    return w @ np.maximum(q @ keys.T, 0.0)


@pytest.mark.parametrize("shared", [0.0, 0.9])
def test_certificate_is_an_upper_bound(shared):
    """Random heads (shared = 0) and heads that share one direction
    (shared = 0.9, the regime the page's bounds are built for)."""
    rng = np.random.default_rng(11)
    for case in range(60):
        H, d = int(rng.integers(2, 40)), int(rng.integers(2, 33))
        base = rng.standard_normal(d)
        q = shared * base + np.sqrt(1 - shared ** 2) * rng.standard_normal((H, d))
        w = rng.standard_normal(H)
        keys = rng.standard_normal((300, d))
        r = int(rng.integers(0, H + 1))
        cert = dosa.certificate(q, w, keys[:64], r)
        U = dosa.upper_bounds(cert, keys)
        s = _scores(q, w, keys)
        assert np.all(U >= s - 1e-9 * (1 + np.abs(s))), (case, float((s - U).max()))


def test_every_head_kept_gives_the_score():
    rng = np.random.default_rng(3)
    q, w, keys = rng.standard_normal((12, 8)), rng.standard_normal(12), rng.standard_normal((50, 8))
    cert = dosa.certificate(q, w, keys, r=12)
    assert cert["E"] == 0.0 and not cert["aA"].any()
    np.testing.assert_allclose(dosa.upper_bounds(cert, keys), _scores(q, w, keys), rtol=1e-12,
                               atol=1e-12)


def test_positive_multiple_folds_exactly():
    """q_1 = 2.5 q_0 with both weights positive and a budget of one head: the
    rule keeps the head with the larger w_h ||q_h|| (head 1: 1.3 x 2.5 > 0.7),
    head 0 projects onto it with beta = 1/2.5 = 0.4 and no residual, so the
    certificate is the score exactly: w~_1 = 1.3 + 0.4 x 0.7, E = 0."""
    rng = np.random.default_rng(4)
    q0 = rng.standard_normal(6)
    q = np.stack([q0, 2.5 * q0])
    w = np.array([0.7, 1.3])
    keys = rng.standard_normal((40, 6))
    cert = dosa.certificate(q, w, keys, r=1)
    assert cert["kept"] == [1] and abs(cert["E"]) < 1e-12
    assert cert["w_fold"][0] == pytest.approx(1.3 + 0.4 * 0.7)
    np.testing.assert_allclose(dosa.upper_bounds(cert, keys), _scores(q, w, keys), rtol=1e-12,
                               atol=1e-12)


def test_without_seeds_negative_heads_rank_by_weighted_norm():
    """An empty seed set: p_h = 1/2 for every head, so with at most r
    positive heads the remaining budget goes to the negative heads of
    largest |w_h| ||q_h||, no head is majority-active, and the bound still
    holds."""
    rng = np.random.default_rng(12)
    H, d = 48, 16
    q = rng.standard_normal((H, d))
    w = rng.standard_normal(H)
    w[:10] = np.abs(w[:10]) + 0.1                      # 10 positive heads ...
    w[10:] = -np.abs(w[10:]) - 0.1                     # ... and 38 negative ones
    cert = dosa.certificate(q, w, np.zeros((0, d)), r=32)
    neg = np.arange(10, H)
    want_neg = neg[np.argsort(-(np.abs(w[neg]) * np.linalg.norm(q[neg], axis=1)),
                              kind="stable")[:22]]
    assert sorted(cert["kept"]) == sorted(list(range(10)) + want_neg.tolist())
    assert cert["E"] == 0.0                            # every positive head is kept
    assert not cert["aA"].any()                        # no activation evidence, A empty
    keys = rng.standard_normal((500, d))
    assert np.all(dosa.upper_bounds(cert, keys) >= _scores(q, w, keys) - 1e-9)


def test_seed_threshold_is_a_lower_bound_of_the_kth_score():
    rng = np.random.default_rng(5)
    s = rng.standard_normal(5000)
    for K in (1, 10, 300):
        for n in (K, 2 * K, 4000):
            seed = rng.choice(5000, size=n, replace=False)
            assert dosa.seed_threshold(s[seed], K) <= np.sort(s)[-K]


def test_survival_on_the_synthetic_workload():
    """Rows of the 256K-query CSA workload (i.i.d. N(0, 1/d) heads and keys,
    r = 32 of 64 heads, seed = the first 2K visible keys): the certificate
    holds on every key and the share of keys it cannot reject is recorded.
    On these inputs nearly every key survives the seed threshold -- the
    pruning the page reports comes from trained head geometry."""
    inp = gen.generate("c4_csa_256k", S=3, T=65536)     # rows are i.i.d.: three suffice
    K = inp.topk
    q = inp.q.float().double().numpy()
    w = inp.w.double().numpy()
    k = inp.k.float().double().numpy()
    out = []
    for t, P in enumerate((8192, 32768, 65536)):          # visible keys of the row
        keys = k[:P]
        s = _scores(q[t], w, keys)
        tau = dosa.seed_threshold(s[:2 * K], K)
        cert = dosa.certificate(q[t], w, keys[:2 * K], r=32)
        U = dosa.upper_bounds(cert, keys)
        assert np.all(U >= s - 1e-9 * (1 + np.abs(s)))
        out.append(((U >= tau).mean(), (s >= tau).mean(), (U >= np.sort(s)[-K]).mean()))
    surv = np.array(out)
    print("survival (certificate vs seed tau, exact score vs seed tau, certificate vs final "
          "K-th score):", np.round(surv, 3).tolist())
    assert surv[:, 0].min() > 0.5      # the screen rejects little on these inputs
