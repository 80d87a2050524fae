"""The seeded generators follow their stated recipe (CPU, scaled-down sizes)."""
import math

import numpy as np
import pytest
import torch

from workloads import gen


@pytest.mark.parametrize("name", gen.config_names())
def test_shapes_dtypes_and_determinism(name):
    a = gen.generate(name, S=256)
    b = gen.generate(name, S=256)
    assert a.q.shape == (256, a.H, a.d) and a.k.shape == (a.T, a.d)
    want = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[a.dtype]
    assert a.q.dtype == want and a.k.dtype == want
    for x, y in ((a.q, b.q), (a.k, b.k), (a.w, b.w)):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.float8_e4m3fn else x,
                           y.view(torch.uint8) if y.dtype == torch.float8_e4m3fn else y)
    if a.dtype == "fp8":
        assert a.q_scale.shape == (256, a.H) and a.k_scale.shape == (a.T,)
    else:
        assert a.q_scale is None and a.k_scale is None


def test_full_size_config_table():
    c = gen.CONFIGS
    assert (c["c1_tiny_int"]["S"], c["c1_tiny_int"]["H"], c["c1_tiny_int"]["d"]) == (1024, 4, 32)
    assert (c["c2_glm_pooled"]["T"], c["c2_glm_pooled"]["m"], c["c2_glm_pooled"]["topk"]) == (8192, 4, 2048)
    assert (c["c3_dsa_token"]["S"], c["c3_dsa_token"]["T"]) == (131072, 131072)
    assert (c["c4_csa_256k"]["S"], c["c4_csa_256k"]["T"], c["c4_csa_256k"]["query_chunk"]) == (262144, 65536, 16384)
    assert (c["c5_csa_1m"]["S"], c["c5_csa_1m"]["T"], c["c5_csa_1m"]["query_chunk"]) == (1048576, 262144, 32768)


def test_fp8_rows_use_amax_over_448():
    a = gen.generate("c3_dsa_token", S=64)
    q = a.q.float()
    amax = q.abs().amax(-1)
    assert torch.all(amax == 448.0)          # the largest element maps to the top code
    k = a.k.float()
    assert torch.all(k.abs().amax(-1) == 448.0)


def test_pooled_keys_are_bf16_means_of_bf16_tokens():
    a = gen.generate("c2_glm_pooled", S=64)
    g = torch.Generator().manual_seed(a.seed + 2)
    tok = (torch.randn((a.T * a.m, a.d), generator=g) / math.sqrt(a.d)).to(torch.bfloat16).float()
    want = tok.view(a.T, a.m, a.d).mean(1).to(torch.bfloat16)
    assert torch.equal(a.k, want)


def test_ar1_queries_are_correlated_along_the_sequence():
    a = gen.generate("c3_dsa_token", S=4096, dtype="f32")
    q = a.q.double().numpy().reshape(4096, -1)
    r = np.mean([np.corrcoef(q[:-1, c], q[1:, c])[0, 1] for c in range(0, q.shape[1], 97)])
    assert 0.85 < r < 0.95
    assert 0.8 / a.d < q.var() < 1.2 / a.d


def test_integer_config_values():
    a = gen.generate("c1_tiny_int")
    assert set(torch.unique(a.q).tolist()) <= set(range(-3, 4))
    assert set(torch.unique(a.w).tolist()) == {-1.0, -0.5, 0.5, 1.0}
    assert a.w.shape == (1024, 4)
