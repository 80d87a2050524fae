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

# every pin below takes the certificate module as an argument, so that
# test_dosa_mutants.py can run the same pins against planted mistakes


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


def test_given_activation_frequencies_replace_the_measured_ones():
    """certificate(..., p=...) takes the activation frequencies as given: the
    measured ones reproduce the default certificate; moving one omitted
    negative head across 1/2 moves it into or out of the majority-active set
    and the aggregate by exactly |w_h| q_h; frequencies without seeds are
    refused."""
    rng = np.random.default_rng(21)
    H, d = 40, 16
    q = rng.standard_normal((H, d))
    w = rng.standard_normal(H)
    seeds = rng.standard_normal((300, d))
    base = dosa.certificate(q, w, seeds, r=20)
    same = dosa.certificate(q, w, seeds, r=20, p=base["p"])
    assert same["kept"] == base["kept"] and same["A"] == base["A"]
    np.testing.assert_array_equal(same["aA"], base["aA"])
    omitted = [h for h in range(H)
               if w[h] < 0 and h not in base["kept"] and base["p"][h] != 0.5]
    assert omitted
    h = omitted[0]
    # p -> 1 - p keeps the priority min(p, 1 - p), so the kept set stays
    p = base["p"].copy()
    p[h] = 1 - p[h]
    moved = dosa.certificate(q, w, seeds, r=20, p=p)
    assert moved["kept"] == base["kept"]
    assert (h in moved["A"]) != (h in base["A"])
    sign = 1.0 if h in moved["A"] else -1.0
    np.testing.assert_allclose(moved["aA"] - base["aA"], sign * abs(w[h]) * q[h], atol=1e-12)
    with pytest.raises(ValueError):
        dosa.certificate(q, w, np.zeros((0, d)), r=20, p=np.full(H, 0.5))


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


# Seeds of the hand-derived cases below (d = 4): the signs of k_y, k_z and
# k_w over the 8 seed keys fix the activation frequencies
# p_1 = 4/8 (head 1 reads k_y), p_2 = 7/8 (head 2 reads k_z), p_3 = 4/8
# (head 3 reads k_w) and p_4 = 1/8 (head 4 reads -k_z).
_SEEDS = np.array([[0, y, z, u] for y, z, u in zip([1, 1, 1, 1, -1, -1, -1, -1],
                                                   [1, 1, 1, 1, 1, 1, 1, -1],
                                                   [1, -1, 1, -1, 1, -1, 1, -1])], float)
_Q4 = np.array([[1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 2, 0], [0, 0, 0, 1], [0, 0, -1, 0]], float)
_W4 = np.array([1.0, -1.0, -1.0, -0.25, -0.1])


def pin_activation_frequency_ranks_negative_heads(mod=dosa):
    """Budget r = 2: head 0 (the only positive head) plus one negative head.
    By |w_h| ||q_h|| alone head 2 (1 x 2) beats head 1 (1 x 1), but the
    page's priority weighs in min(p_h, 1 - p_h): head 1 gets 1 x 1 x 1/2 =
    0.5, head 2 gets 1 x 2 x 1/8 = 0.25, head 3 0.25 x 1 x 1/2 = 0.125,
    head 4 0.1 x 1 x 1/8 = 0.0125 -- so heads 0 and 1 are kept."""
    cert = mod.certificate(_Q4, _W4, _SEEDS, r=2)
    # k_x = 0 on every seed: head 0 never fires
    np.testing.assert_allclose(cert["p"], [0.0, 0.5, 7 / 8, 0.5, 1 / 8])
    assert sorted(cert["kept"]) == [0, 1]


def pin_majority_active_aggregate_by_hand(mod=dosa):
    """Same row: the omitted negative heads are 2 (p = 7/8), 3 (p = 1/2, on
    the boundary, included since A takes p_h >= 1/2) and 4 (p = 1/8, left
    out), so a_A = 1 x (0,0,2,0) + 0.25 x (0,0,0,1) = (0,0,2,0.25).  For the
    key (1,0,1,4): kept part 1 x [1]_+ + (-1) x [0]_+ = 1, aggregate
    [2 + 1]_+ = 3, U = 1 - 3 = -2, which is the exact score
    1 - 0 - 1 x 2 - 0.25 x 4 - 0.1 x [-1]_+ = -2.  For (1,0,-1,-4) the
    aggregate is [-3]_+ = 0 and U = 1 against the score 1 - 0.1 x 1 = 0.9.
    Without the aggregate U would be 1 for both; with head 4 in A it would
    be -1.9 for the first key."""
    cert = mod.certificate(_Q4, _W4, _SEEDS, r=2)
    assert sorted(cert["A"]) == [2, 3]
    np.testing.assert_allclose(cert["aA"], [0, 0, 2, 0.25])
    keys = np.array([[1, 0, 1, 4], [1, 0, -1, -4]], float)
    np.testing.assert_allclose(mod.upper_bounds(cert, keys), [-2.0, 1.0], atol=1e-12)
    np.testing.assert_allclose(_scores(_Q4, _W4, keys), [-2.0, 0.9], atol=1e-12)


def _joint_case(q_omit, w_omit):
    """Head 0 = (3,0,0) kept (largest w ||q||, budget 1), the given omitted
    positive heads orthogonal to it (beta = 0, residual = the head)."""
    q = np.vstack([[3.0, 0, 0], q_omit])
    w = np.concatenate([[1.0], w_omit])
    return q, w


def pin_joint_residual_closed_forms(mod=dosa):
    """u_h = w_h q_h here.  Orthogonal residuals u = (0,1,0), (0,0,0.5):
    ||sum u|| = sqrt(1.25) and sum |u_h . u_l| = 1.25, so E_joint =
    sqrt(1.25) = sqrt(5)/2 against E = 1.5.  Parallel u = (0,1,0), (0,1,0):
    E_joint = (2 + sqrt(4)) / 2 = 2 = E.  Opposite u = (0,1,0), (0,-1,0):
    E_joint = (0 + sqrt(4)) / 2 = 1 against E = 2, and it is attained:
    [k_y]_+ + [-k_y]_+ = |k_y| = 1 x ||k|| at k = (0,1,0)."""
    q, w = _joint_case([[0, 1, 0], [0, 0, 1]], [1.0, 0.5])
    c = mod.certificate(q, w, np.zeros((0, 3)), r=1)
    assert c["E"] == pytest.approx(1.5) and c["E_joint"] == pytest.approx(np.sqrt(5) / 2)
    q, w = _joint_case([[0, 1, 0], [0, 2, 0]], [1.0, 0.5])
    c = mod.certificate(q, w, np.zeros((0, 3)), r=1)
    assert c["E"] == pytest.approx(2.0) and c["E_joint"] == pytest.approx(2.0)
    q, w = _joint_case([[0, 1, 0], [0, -1, 0]], [1.0, 1.0])
    c = mod.certificate(q, w, np.zeros((0, 3)), r=1)
    assert c["E"] == pytest.approx(2.0) and c["E_joint"] == pytest.approx(1.0)
    k = np.array([[0.0, 1.0, 0.0]])
    assert mod.upper_bounds(c, k)[0] == pytest.approx(_scores(q, w, k)[0])   # tight


def pin_projection_clips_negative_correlation(mod=dosa):
    """Kept head 0 = (1,0) (w = 2), omitted positive head 1 = (-1,1) (w = 1):
    q_1 . q_0 = -1, so beta = [-1]_+ / 1 = 0, no fold, residual = q_1 and
    E = E_joint = sqrt(2).  At k = (-1,1) the score is 2 x 0 + 1 x [2]_+ = 2
    and U = 0 + sqrt(2) x sqrt(2) = 2 (tight); an unclipped beta = -1 would
    fold w_0 to 1 and claim U = sqrt(2) < 2."""
    q = np.array([[1.0, 0.0], [-1.0, 1.0]])
    w = np.array([2.0, 1.0])
    c = mod.certificate(q, w, np.zeros((0, 2)), r=1)
    assert c["kept"] == [0] and c["w_fold"][0] == pytest.approx(2.0)
    assert c["E_joint"] == pytest.approx(np.sqrt(2))
    k = np.array([[-1.0, 1.0]])
    assert mod.upper_bounds(c, k)[0] == pytest.approx(2.0)


def pin_bounds_hold_on_random_rows(mod=dosa):
    """U >= s with the joint and with the per-head allowance, on random rows
    with and without seeds (a_A in play), shared and independent heads."""
    rng = np.random.default_rng(21)
    for case in range(80):
        H, d = int(rng.integers(2, 40)), int(rng.integers(2, 24))
        shared = 0.9 if case % 2 else 0.0
        q = shared * rng.standard_normal(d) + np.sqrt(1 - shared ** 2) * \
            rng.standard_normal((H, d))
        w = rng.standard_normal(H)
        keys = rng.standard_normal((200, d))
        c = mod.certificate(q, w, keys[:int(rng.integers(0, 64))], int(rng.integers(0, H + 1)))
        s = _scores(q, w, keys)
        assert c["E_joint"] <= c["E"] * (1 + 1e-12) + 1e-12
        for joint in (True, False):
            U = mod.upper_bounds(c, keys, joint=joint)
            assert np.all(U >= s - 1e-9 * (1 + np.abs(s))), (case, joint)


DOSA_PINS = [pin_activation_frequency_ranks_negative_heads, pin_majority_active_aggregate_by_hand,
             pin_joint_residual_closed_forms, pin_projection_clips_negative_correlation,
             pin_bounds_hold_on_random_rows]


@pytest.mark.parametrize("pin", DOSA_PINS, ids=lambda f: f.__name__)
def test_dosa_pin(pin):
    pin()
