"""Parity of the HIP path (called through the C ABI) with the CPU oracle.

Integer-exact problems must match bit for bit; float problems follow the
tolerance rule in oracle/check.py.  Scaled-down problems are compared on
every row (several key tiles, compactions and a ragged last tile); the five
full-size workloads run in the launch configuration the benchmark times and
are compared on sampled rows, with the all-row invariants checked on the
device.
"""
import numpy as np
import pytest
import torch

from gpu_util import device_invariants, log, rows_to_host, run
from oracle import check
from oracle import oracle as orc
from workloads import gen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _compare_all(inp, out, exact=None):
    idx, vl, sc = out
    rows = np.arange(inp.S)
    rep = check.compare(inp, rows, idx.cpu().numpy(), vl.cpu().numpy(),
                        None if sc is None else sc.cpu().numpy(), exact=exact)
    assert rep["ok"], rep["failures"]
    return rep


def test_c1_integer_exact_all_rows():
    inp = gen.generate("c1_tiny_int").to(DEV)
    log(f"c1 full S={inp.S}")
    out = run(inp)
    rep = _compare_all(inp, out, exact=True)
    assert rep["exact"]
    device_invariants(inp, out[0], out[1])


SCALED = [
    ("c1_tiny_int", 3001, 64),     # ragged: S, T not multiples of the tile sizes
    ("c2_glm_pooled", 4096, 512),  # 128 pools of 1024 visible: compactions + tail
    ("c2_glm_pooled", 1000, 64),
    ("c3_dsa_token", 4096, 256),   # fp8 with scales, AR(1) queries
    ("c4_csa_256k", 8192, 256),    # bf16 compressed keys
    ("c5_csa_1m", 6000, 128),      # fp8 compressed keys, ragged
]


@pytest.mark.parametrize("name,S,topk", SCALED)
def test_scaled_configs_all_rows(name, S, topk):
    inp = gen.generate(name, S=S, topk=topk).to(DEV)
    log(f"{name} S={S} T={inp.T} topk={topk}")
    out = run(inp, query_chunk=0)
    rep = _compare_all(inp, out)
    log(f"  index-mismatch rows {rep['index_mismatch_rows']}, max score rel err "
        f"{rep['max_score_rel_err']:.2e}")
    device_invariants(inp, out[0], out[1])


FULL = ["c2_glm_pooled", "c3_dsa_token", "c4_csa_256k", "c5_csa_1m"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_rows(name):
    inp = gen.generate(name, device=DEV)
    log(f"{name} full S={inp.S} T={inp.T} H={inp.H} d={inp.d} dtype={inp.dtype} "
        f"chunk={inp.query_chunk}")
    idx, vl, sc = run(inp)
    device_invariants(inp, idx, vl)
    ksel = inp.topk // inp.m if inp.expand else inp.topk
    n_uniform = 320 if inp.S >= 1 << 20 else 640
    rows = check.sample_rows(inp.S, m=inp.m, ksel=ksel, chunk=inp.query_chunk, seed=inp.seed,
                             n_uniform=n_uniform)
    hi, hv, hs = rows_to_host(rows, idx, vl, sc)
    rep = check.compare(inp, rows, hi, hv, hs)
    log(f"  rows {rep['rows']}, index-mismatch rows {rep['index_mismatch_rows']}, "
        f"max score rel err {rep['max_score_rel_err']:.2e}")
    assert rep["ok"], rep["failures"]
    # the benchmark's call asks for no scores (rows that see at most Ksel
    # keys are then written unscored): the same rows, bit for bit
    del sc
    idx2, vl2 = run(inp, with_scores=False)
    assert torch.equal(vl, vl2) and torch.equal(idx, idx2)


def test_c2_every_row_at_full_size():
    """The 32K-token pooled workload (expansion and tail, 2,051-slot rows)
    at full size: every one of its 32,768 rows against the oracle, not a
    sample (about 4.3e9 triples of fp64 oracle work)."""
    inp = gen.generate("c2_glm_pooled", device=DEV)
    idx, vl, sc = run(inp)
    rows = np.arange(inp.S)
    rep = check.compare(inp, rows, idx.cpu().numpy(), vl.cpu().numpy(), sc.cpu().numpy())
    log(f"  rows {rep['rows']}, index-mismatch rows {rep['index_mismatch_rows']}, "
        f"max score rel err {rep['max_score_rel_err']:.2e}")
    assert rep["ok"], rep["failures"][:3]


def test_full_size_query_chunk_sweep_is_bit_identical():
    """The StreamIndex abstract's chunk sweep at the 256K-query workload's
    full size: query chunks of 4K, 8K, 16K (the benchmark's) and 32K rows
    give the same rows bit for bit (rows are independent; only the launch
    sizes differ)."""
    inp = gen.generate("c4_csa_256k", device=DEV)
    ref = run(inp, with_scores=False, query_chunk=16384)
    for chunk in (4096, 8192, 32768):
        out = run(inp, with_scores=False, query_chunk=chunk)
        assert torch.equal(out[1], ref[1]) and torch.equal(out[0], ref[0]), chunk


@pytest.mark.parametrize("topk", [512, 1024, 4096])
def test_full_size_topk_sweep_sampled_rows(topk):
    """The abstract's top-k sweep at the 256K-query workload's full size (the
    benchmark's 2048 is covered above): sampled rows against the oracle, and
    every row's invariants on the device."""
    inp = gen.generate("c4_csa_256k", topk=topk, device=DEV)
    idx, vl, sc = run(inp)
    device_invariants(inp, idx, vl)
    rows = check.sample_rows(inp.S, m=inp.m, ksel=topk, chunk=inp.query_chunk, seed=inp.seed,
                             n_uniform=64)
    hi, hv, hs = rows_to_host(rows, idx, vl, sc)
    rep = check.compare(inp, rows, hi, hv, hs)
    log(f"  topk {topk}: rows {rep['rows']}, index-mismatch rows {rep['index_mismatch_rows']}, "
        f"max score rel err {rep['max_score_rel_err']:.2e}")
    assert rep["ok"], rep["failures"]


def test_automatic_query_chunk_is_bit_identical():
    """query_chunk = 0 takes as many rows per launch as 4 GiB of candidate
    buffers hold (25,888 at the 256K workload): the same rows as the
    benchmark's 16,384-row chunks, bit for bit."""
    inp = gen.generate("c4_csa_256k", device=DEV)
    a = run(inp, with_scores=False)
    b = run(inp, with_scores=False, query_chunk=0)
    assert torch.equal(a[1], b[1]) and torch.equal(a[0], b[0])


# ---------------------------------------------------------------- edge cases
def _exact_rows(inp, out):
    ref = orc.select_rows(inp, np.arange(inp.S))
    assert np.array_equal(out[1].cpu().numpy(), ref["valid_len"])
    assert np.array_equal(out[0].cpu().numpy(), ref["idx"])
    return ref


def test_worked_examples_on_gpu():
    # WE1 / WE2: signed weights, an all-ReLU-zero key, and the tie rule (d padded to 32)
    q = torch.zeros(5, 2, 32)
    q[:, 0, 0] = 1
    q[:, 1, 1] = 1
    k = torch.zeros(5, 32)
    k[:, :2] = torch.tensor([[2., 1.], [1., 3.], [-1., -1.], [3., -2.], [1., 1.]])
    w = torch.tensor([1.0, -1.0])
    for topk in (2, 3):
        inp = gen.custom(q=q, k=k, w=w, topk=topk).to(DEV)
        out = run(inp)
        _exact_rows(inp, out)
    assert out[0][4].tolist() == [0, 2, 3]
    # WE4: pool [4..7] is never visible to query 5
    q = torch.ones(9, 1, 32)
    k = torch.zeros(2, 32)
    k[0, 0], k[1, 0] = 1.0, 2.0
    inp = gen.custom(q=q, k=k, w=torch.ones(1), m=4, topk=4, expand=True, tail=True).to(DEV)
    out = run(inp)
    _exact_rows(inp, out)
    assert out[0][5].tolist() == [0, 1, 2, 3, 4, 5, -1]
    assert out[0][7].tolist() == [4, 5, 6, 7, -1, -1, -1]


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5, 7, 8, 9, 63, 64, 65])
def test_watch_lengths_pooled_tail(S):
    inp = gen.generate("c2_glm_pooled", S=max(S, 4), topk=8)
    inp = gen.custom(q=inp.q[:S], k=inp.k[:max(1, S // 4)], w=inp.w, m=4, topk=8, expand=True,
                     tail=True).to(DEV)
    out = run(inp)
    _compare_all(inp, out)
    device_invariants(inp, out[0], out[1])


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
def test_all_scores_tie(dtype):
    """q = 0: every score is 0; the tie rule keeps the lowest indices, through
    many compactions whose cut falls inside one run of equal codes."""
    S = T = 3000
    H, d = 64, 64
    g = torch.Generator().manual_seed(5)
    k = torch.randn(T, d, generator=g)
    q = torch.zeros(S, H, d)
    w = torch.randn(H, generator=g)
    q_scale = k_scale = None
    if dtype == "bf16":
        q, k = q.bfloat16(), k.bfloat16()
    elif dtype == "fp8":
        q, q_scale = gen.quant_e4m3_rows(q)
        k, k_scale = gen.quant_e4m3_rows(k)
    inp = gen.custom(q=q, k=k, w=w, topk=100, q_scale=q_scale, k_scale=k_scale).to(DEV)
    idx, vl, sc = run(inp)
    want = np.full((S, 100), -1, np.int32)
    for t in range(S):
        n = min(100, t + 1)
        want[t, :n] = np.arange(n)
    assert np.array_equal(idx.cpu().numpy(), want)
    assert bool((sc == 0).all())


def test_all_relu_zero_rows():
    """Every q.k negative: every ReLU is 0, every score 0."""
    S = T = 700
    q = -torch.ones(S, 4, 32)
    k = torch.rand(T, 32, generator=torch.Generator().manual_seed(2)) + 0.1
    inp = gen.custom(q=q, k=k, w=torch.tensor([1.0, -0.5, 2.0, -1.0]), topk=50).to(DEV)
    out = run(inp)
    _exact_rows(inp, out)


@pytest.mark.parametrize("order", ["ascending", "descending"])
def test_monotone_scores(order):
    """Ascending scores make every key beat the running threshold (maximal
    compaction work); descending ones make the threshold reject everything
    after the first fill."""
    S = T = 5000
    q = torch.zeros(S, 1, 32)
    q[:, 0, 0] = 1.0
    k = torch.zeros(T, 32)
    k[:, 0] = torch.arange(T, dtype=torch.float32) * (1 if order == "ascending" else -1)
    inp = gen.custom(q=q, k=k, w=torch.ones(1), topk=300).to(DEV)
    out = run(inp)
    ref = _exact_rows(inp, out)
    t = S - 1
    want = np.arange(T - 300, T) if order == "ascending" else np.arange(300)
    assert np.array_equal(ref["idx"][t], want)


def test_topk_larger_than_visible_and_topk_one():
    base = gen.generate("c4_csa_256k", S=2048).to(DEV)
    for topk in (1, 4096):
        inp = gen.custom(q=base.q, k=base.k, w=base.w, m=4, topk=topk).to(DEV)
        out = run(inp)
        _compare_all(inp, out)
        device_invariants(inp, out[0], out[1])


@pytest.mark.parametrize("causal,q_pos0", [(True, 15988), (False, 0)])
def test_largest_supported_topk_on_both_paths(causal, q_pos0):
    """topk = 16,000, the largest Ksel the library takes (its 16-bit
    histogram counters bound a candidate buffer below 65,536 entries):
    causal rows that see from 15,989 to 16,012 keys (fewer than, exactly and
    more than Ksel), and non-causal rows that see all 40,000 keys.  Every row
    against the oracle, on the streaming path and on the few-query path --
    whose cut list holds 8,192 candidates, so these rows reach the result
    through its repair launch -- and the two paths bit for bit."""
    g = torch.Generator().manual_seed(16000)
    S, H, d, T = 24, 8, 64, 40000
    q = (torch.randn(S, H, d, generator=g) / d ** 0.5).bfloat16()
    k = (torch.randn(T, d, generator=g) / d ** 0.5).bfloat16()
    w = torch.randn(H, generator=g)
    inp = gen.custom(q=q, k=k, w=w, topk=16000, causal=causal, q_pos0=q_pos0).to(DEV)
    stream = run(inp)
    few = run(inp, few_query_rows=64)
    for x, y in zip(stream, few):
        assert torch.equal(x, y)
    _compare_all(inp, stream)
    device_invariants(inp, stream[0], stream[1])
    vl = stream[1].cpu()
    want = torch.clamp(torch.arange(S) + q_pos0 + 1, max=16000) if causal else torch.full((S,), 16000)
    assert torch.equal(vl, want.int())


@pytest.mark.parametrize("expand,tail,causal,q_pos0,T", [
    (False, False, True, 0, None),       # first 2048 pools' rows taken whole
    (True, True, True, 6001, None),      # blocks straddle the Ksel edge
    (False, False, False, 0, 2000),      # non-causal, every row sees T <= Ksel
    (True, False, False, 0, 3000)])      # non-causal, T > Ksel: scored
def test_rows_with_at_most_ksel_keys_need_no_scores(expand, tail, causal, q_pos0, T):
    """A row that sees at most Ksel keys selects all of them, so without
    sel_score a block of such rows writes them without scoring; the result
    equals the scored path's bit for bit and passes the oracle's rule."""
    base = gen.generate("c4_csa_256k", S=12000, T=T or 4600)
    inp = gen.custom(q=base.q, k=base.k, w=base.w, m=4, topk=2048 * (4 if expand else 1),
                     expand=expand, tail=tail, causal=causal, q_pos0=q_pos0).to(DEV)
    idx, vl, sc = run(inp, with_scores=True)
    idx2, vl2 = run(inp, with_scores=False)
    assert torch.equal(idx, idx2) and torch.equal(vl, vl2)
    device_invariants(inp, idx2, vl2)
    rows = np.concatenate([np.arange(0, inp.S, 97), [inp.S - 1]])
    rep = check.compare(inp, rows, idx2.cpu().numpy()[rows], vl2.cpu().numpy()[rows])
    assert rep["ok"], rep["failures"][:3]


def test_non_causal_and_ragged():
    base = gen.generate("c4_csa_256k", S=1001, T=777, topk=100)
    inp = gen.custom(q=base.q, k=base.k, w=base.w, m=4, topk=100, causal=False).to(DEV)
    out = run(inp)
    _compare_all(inp, out)
    assert bool((out[1] == 100).all())


def test_empty_inputs():
    base = gen.generate("c4_csa_256k", S=64).to(DEV)
    inp = gen.custom(q=base.q[:0], k=base.k, w=base.w, m=4, topk=16).to(DEV)
    idx, vl, _ = run(inp)
    assert idx.shape == (0, 16) and vl.shape == (0,)
    inp = gen.custom(q=base.q, k=base.k[:0], w=base.w, m=4, topk=16).to(DEV)
    idx, vl, _ = run(inp)
    assert bool((vl == 0).all()) and bool((idx == -1).all())
    # tail only: no complete pool for the first three positions
    inp = gen.custom(q=base.q[:3], k=base.k[:0], w=base.w, m=4, topk=16, expand=True,
                     tail=True).to(DEV)
    idx, vl, _ = run(inp)
    assert vl.tolist() == [1, 2, 3]
    assert idx[2, :4].tolist() == [0, 1, 2, -1]


@pytest.mark.parametrize("dtype,H,d", [("bf16", 4, 64), ("bf16", 16, 128), ("bf16", 33, 32),
                                       ("bf16", 64, 64), ("fp8", 32, 64), ("fp8", 48, 128),
                                       ("f32", 48, 64), ("f32", 64, 32)])
def test_head_and_dim_variants(dtype, H, d):
    S, T = 1500, 1500
    g = torch.Generator().manual_seed(H * 1000 + d)
    q = torch.randn(S, H, d, generator=g) / d ** 0.5
    k = torch.randn(T, d, generator=g) / d ** 0.5
    w = torch.randn(S, H, generator=g)                # per-row weights
    q_scale = k_scale = None
    if dtype == "bf16":
        q, k = q.bfloat16(), k.bfloat16()
    elif dtype == "fp8":
        q, q_scale = gen.quant_e4m3_rows(q)
        k, k_scale = gen.quant_e4m3_rows(k)
    inp = gen.custom(q=q, k=k, w=w, topk=96, q_scale=q_scale, k_scale=k_scale).to(DEV)
    out = run(inp)
    _compare_all(inp, out)


def test_chunking_q_pos0_and_determinism_are_bit_identical():
    inp = gen.generate("c4_csa_256k", S=12000, topk=256).to(DEV)
    ref = run(inp, query_chunk=0)
    for chunk in (1000, 4096, 7777):
        out = run(inp, query_chunk=chunk)
        for a, b in zip(ref, out):
            assert torch.equal(a, b), f"chunk {chunk}"
    again = run(inp, query_chunk=0)
    for a, b in zip(ref, again):
        assert torch.equal(a, b)
    # external chunking: rows [a, S) called alone at q_pos0 = a
    a = 5000
    sub = gen.custom(q=inp.q[a:], k=inp.k, w=inp.w, m=4, topk=256, q_pos0=a)
    out = run(sub, query_chunk=0)
    for x, y in zip(ref, out):
        assert torch.equal(x[a:], y)


def test_pair_overlap_matches_oracle():
    inp = gen.generate("c3_dsa_token", S=6001, topk=256).to(DEV)
    import dsa_indexer_score_amd as dsai
    idx, vl, _ = run(inp)
    shared = dsai.pair_overlap(idx, vl)
    torch.cuda.synchronize()
    hi, hv = idx.cpu().numpy(), vl.cpu().numpy()
    want = orc.pair_overlap(hi, hv)
    assert np.array_equal(shared.cpu().numpy(), want)
    st = dsai.overlap_summary(shared, vl)
    ref = orc.overlap_stats(want, hv)
    assert st["pairs"] == ref["pairs"]
    assert st["mean_overlap"] == pytest.approx(ref["mean_overlap"], rel=1e-12)
    assert st["p90_overlap"] == pytest.approx(ref["p90_overlap"], rel=1e-12)
    log(f"  AR(1) fp8 adjacent-pair overlap: mean {st['mean_overlap']:.3f}, "
        f"median {st['median_overlap']:.3f}")
    # causal prefix pairs (rows 2i, 2i+1 with t < topk) overlap completely
    assert (want[:100] == hv[0:200:2]).all()


@pytest.mark.parametrize("W", [2051, 5000])
def test_pair_overlap_wide_ranges_and_ragged_rows(W):
    """Rows whose index range spans several bitmap windows (up to 400,000),
    ragged and empty valid lengths, an odd row count, shared and disjoint
    entries, rows short enough to sit in registers and rows longer than that
    -- against the oracle's exact set intersection."""
    import dsa_indexer_score_amd as dsai
    rng = np.random.default_rng(11 + W)
    S = 301
    idx = np.full((S, W), -1, np.int32)
    vl = np.zeros(S, np.int32)
    for t in range(S):
        span = int(rng.choice([50, 5000, 140000, 400000]))
        n = int(rng.choice([0, 1, 63, 64, 65, 1000, 2400, W])) if t % 7 else 0
        n = min(n, span, W)
        if t % 2 == 1 and vl[t - 1] > 0 and rng.random() < 0.7:
            prev = idx[t - 1, :vl[t - 1]]            # overlap with the partner row
            keep = prev[rng.random(prev.size) < 0.5]
            extra = rng.choice(span, size=n, replace=False)
            row = np.unique(np.concatenate([keep, extra]))[:W]
        else:
            row = np.sort(rng.choice(span, size=n, replace=False))
        idx[t, :row.size] = row
        vl[t] = row.size
    d_idx = torch.from_numpy(idx).to(DEV)
    d_vl = torch.from_numpy(vl).to(DEV)
    shared = dsai.pair_overlap(d_idx, d_vl)
    torch.cuda.synchronize()
    want = orc.pair_overlap(idx, vl)
    assert shared.shape[0] == S // 2
    assert np.array_equal(shared.cpu().numpy(), want)
    assert want.max() > 0 and (want == 0).any()
    if W > 2304:
        assert (vl > 2304).any()
    # 150 pairs take the block-per-pair kernel; the same pairs repeated into a
    # batch of 600 take the wave-per-pair kernel
    big = torch.from_numpy(np.tile(idx[:300], (4, 1))).to(DEV)
    big_vl = torch.from_numpy(np.tile(vl[:300], 4)).to(DEV)
    shared4 = dsai.pair_overlap(big, big_vl)
    assert np.array_equal(shared4.cpu().numpy(), np.tile(want[:150], 4))


@pytest.mark.parametrize("W", [2051, 2304, 2305])
def test_pair_regions_skewed_pairs(W):
    """Skewed pairs -- a dense block of row B inside a short stretch of a
    sparse row A spanning 2.2M positions (34 bitmap windows, most holding
    entries of one row only), equal rows, rows shifted by one, an empty
    row -- at widths on both sides of the register path's limit (2304
    entries per row): exact against the oracle."""
    import dsa_indexer_score_amd as dsai
    n = min(W, 2200)
    A = np.arange(n, dtype=np.int64) * 1000                     # sparse, ascending
    B = 333_333 + np.arange(n, dtype=np.int64)                 # dense block inside one chunk
    B = np.unique(np.concatenate([B[: n - 3], A[[5, 900, n - 1]]]))[:n]
    pairs = [(A, B), (A, A), (A, A + 1), (A, np.zeros(0, np.int64)),
             (np.zeros(0, np.int64), B), (np.arange(W), np.arange(1, W + 1))]
    idx = np.full((2 * len(pairs), W), -1, np.int32)
    vl = np.zeros(2 * len(pairs), np.int32)
    for p_, (x, y) in enumerate(pairs):
        x, y = x[:W], y[:W]
        idx[2 * p_, :x.size], vl[2 * p_] = x, x.size
        idx[2 * p_ + 1, :y.size], vl[2 * p_ + 1] = y, y.size
    got = dsai.pair_regions(torch.from_numpy(idx).to(DEV), torch.from_numpy(vl).to(DEV))
    want = orc.pair_regions(idx, vl)
    for g, w_ in zip(got, want):
        assert np.array_equal(g.cpu().numpy(), w_)


@pytest.mark.parametrize("W", [2051, 5000])
def test_pair_regions_match_oracle(W):
    """The three-region q-cluster split (shared / left-only / right-only with
    device counts) on rows spanning several bitmap windows, ragged and empty
    rows and rows longer than the register path, then on indexer output."""
    import dsa_indexer_score_amd as dsai
    rng = np.random.default_rng(23 + W)
    S = 201
    idx = np.full((S, W), -1, np.int32)
    vl = np.zeros(S, np.int32)
    for t in range(S):
        span = int(rng.choice([50, 5000, 140000, 400000]))
        n = min(int(rng.choice([0, 1, 63, 64, 65, 1000, 2400, W])), span, W)
        if t % 2 == 1 and vl[t - 1] > 0 and rng.random() < 0.7:
            prev = idx[t - 1, :vl[t - 1]]
            row = np.unique(np.concatenate([prev[rng.random(prev.size) < 0.6],
                                            rng.choice(span, size=n, replace=False)]))[:W]
        else:
            row = np.sort(rng.choice(span, size=n, replace=False))
        idx[t, :row.size] = row
        vl[t] = row.size
    got = dsai.pair_regions(torch.from_numpy(idx).to(DEV), torch.from_numpy(vl).to(DEV))
    want = orc.pair_regions(idx, vl)
    for g, w_ in zip(got, want):
        assert np.array_equal(g.cpu().numpy(), w_)
    inp = gen.generate("c3_dsa_token", S=3001, topk=256).to(DEV)
    idx_d, vl_d, _ = run(inp)
    got = dsai.pair_regions(idx_d, vl_d)
    want = orc.pair_regions(idx_d.cpu().numpy(), vl_d.cpu().numpy())
    for g, w_ in zip(got, want):
        assert np.array_equal(g.cpu().numpy(), w_)
    shared = dsai.pair_overlap(idx_d, vl_d)
    assert torch.equal(shared, got[3][:, 0])


def test_fp8_every_code_is_widened_exactly():
    """Each of the 254 finite e4m3 codes, read through the kernel's widening
    and contraction, reproduces the oracle's hand-decoded value exactly:
    with heads (q, -q), weights (+1, -1) and one-hot keys, score_j = q_j."""
    codes = torch.arange(256, dtype=torch.int32)
    codes[(codes & 0x7F) == 0x7F] = 0
    codes = codes.to(torch.uint8)
    q8 = torch.zeros(2, 2, 128, dtype=torch.uint8)
    for t in range(2):
        q8[t, 0] = codes[128 * t:128 * (t + 1)]
        q8[t, 1] = codes[128 * t:128 * (t + 1)] ^ 0x80
    k8 = torch.zeros(128, 128, dtype=torch.uint8)
    k8[torch.arange(128), torch.arange(128)] = 0x38          # 1.0
    inp = gen.custom(q=q8.view(torch.float8_e4m3fn), k=k8.view(torch.float8_e4m3fn),
                     w=torch.tensor([1.0, -1.0]), topk=128, causal=False,
                     q_scale=torch.ones(2, 2), k_scale=torch.ones(128)).to(DEV)
    out = run(inp)
    rep = _compare_all(inp, out, exact=True)
    assert rep["exact"]
    want = np.array([orc.decode_e4m3(int(c)) for c in codes], np.float64).reshape(2, 128)
    assert np.array_equal(out[2].cpu().numpy().astype(np.float64), want + 0.0)
