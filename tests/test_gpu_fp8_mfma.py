"""The e4m3 workloads contracted on the gfx950 fp8 MFMA (IDX_FP8_MFMA)
against the fp64 oracle: the committed evidence for keeping it opt-in.

The fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) sums its 64 products at
reduced internal precision, so its scores are not the fp32-accumulated ones
of the default path (e4m3 widened exactly to bf16).  Measured on MI355X:
its selections meet the fp8 workloads' index rule (oracle/check.py: keys
may differ from the oracle's only within 1e-3 of the k-th score) on every
row of scaled-down problems and on sampled rows of the 128K-token and
1M-token workloads at full size; its reported scores do not meet the score
rule (within 1e-3 of the dequantised oracle's, relative to the score or,
near zero, to 1e-3 of the row's largest selected score) -- measured errors
of 2e-2 to 5e-2 of that scale on scaled-down rows and 6e-3 to 1.2e-2 on the
full-size samples, against about 2e-4 for the default path.  So the default widens, and this instance is a switch for
callers who need indices only.  The tests pin both halves of that, and that
its few-query and streaming paths agree bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_util import device_invariants, log, rows_to_host, run
from oracle import check
from workloads import gen

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _score_err(inp, rows, idx, vl, sc):
    """Largest |s - s*| / max(|s*|, eps_t) over the selected keys of the rows
    (the quantity the score rule bounds by 1e-3)."""
    rep = check.compare(inp, rows, idx, vl, sc)
    return rep["max_score_rel_err"]


@pytest.mark.parametrize("name,S,topk", [("c3_dsa_token", 4096, 256), ("c5_csa_1m", 6000, 128),
                                         ("c3_dsa_token", 2500, 2048)])
def test_fp8_mfma_selections_meet_the_index_rule(name, S, topk):
    inp = gen.generate(name, S=S, topk=topk).to(DEV)
    idx, vl, sc = run(inp, query_chunk=0, fp8_mfma=True)
    rows = np.arange(inp.S)
    idx, vl, sc = idx.cpu().numpy(), vl.cpu().numpy(), sc.cpu().numpy()
    rep = check.compare(inp, rows, idx, vl, None)          # indices and lengths only
    assert rep["ok"], rep["failures"]
    err_fp8 = _score_err(inp, rows, idx, vl, sc)
    d_idx, d_vl, d_sc = run(inp, query_chunk=0)             # the default, widened codes
    err_default = _score_err(inp, rows, d_idx.cpu().numpy(), d_vl.cpu().numpy(),
                             d_sc.cpu().numpy())
    log(f"  {name} S={S} topk={topk}: index-mismatch rows {rep['index_mismatch_rows']}, "
        f"max score rel err fp8 MFMA {err_fp8:.2e}, widened {err_default:.2e}")
    assert err_default <= 1e-3 < err_fp8 < 0.1
    device_invariants(inp, torch.as_tensor(idx, device=DEV), torch.as_tensor(vl, device=DEV))


@pytest.mark.parametrize("name", ["c3_dsa_token", "c5_csa_1m"])
def test_fp8_mfma_full_size_sampled_rows(name):
    inp = gen.generate(name, device=DEV)
    log(f"{name} full S={inp.S} T={inp.T} chunk={inp.query_chunk}, fp8 MFMA")
    idx, vl, sc = run(inp, fp8_mfma=True)
    device_invariants(inp, idx, vl)
    rows = check.sample_rows(inp.S, m=inp.m, ksel=inp.topk, chunk=inp.query_chunk,
                             seed=inp.seed, n_uniform=96 if inp.S >= 1 << 20 else 160)
    hi, hv, hs = rows_to_host(rows, idx, vl, sc)
    rep = check.compare(inp, rows, hi, hv, None)
    err = _score_err(inp, rows, hi, hv, hs)
    log(f"  rows {rep['rows']}, index-mismatch rows {rep['index_mismatch_rows']}, "
        f"extra keys {rep['extra_keys']}, max score rel err {err:.2e}")
    assert rep["ok"], rep["failures"]
    assert err < 0.1


@pytest.mark.parametrize("name,S,T", [("c5_csa_1m", 1, 262144), ("c5_csa_1m", 2, 262144),
                                      ("c3_dsa_token", 40, 131072)])
def test_fp8_mfma_few_query_equals_streaming(name, S, T):
    from dataclasses import replace
    inp = gen.generate(name, S=S, T=T)
    inp = replace(inp, q_pos0=T * inp.m - S).to(DEV)
    a = run(inp, few_query_rows=max(64, S), fp8_mfma=True)
    b = run(inp, few_query_rows=-1, fp8_mfma=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_fp8_mfma_d64_and_missing_heads():
    """d = 64 (one operand per lane half) and H = 40 (a partly empty second
    head block) against the oracle on every row."""
    g = torch.Generator().manual_seed(64)
    S, T, H, d = 600, 3000, 40, 64
    q = torch.randn(S, H, d, generator=g) / d ** 0.5
    k = torch.randn(T, d, generator=g) / d ** 0.5
    qs = q.abs().amax(-1) / 448
    ks = k.abs().amax(-1) / 448
    q8 = (q / qs[..., None]).to(torch.float8_e4m3fn)
    k8 = (k / ks[:, None]).to(torch.float8_e4m3fn)
    inp = gen.custom(q=q8, k=k8, w=torch.randn(H, generator=g), topk=100, q_scale=qs,
                     k_scale=ks, q_pos0=T - S).to(DEV)
    idx, vl, sc = run(inp, fp8_mfma=True)
    rep = check.compare(inp, np.arange(S), idx.cpu().numpy(), vl.cpu().numpy(), None)
    assert rep["ok"], rep["failures"]
    assert _score_err(inp, np.arange(S), idx.cpu().numpy(), vl.cpu().numpy(),
                      sc.cpu().numpy()) < 0.1
