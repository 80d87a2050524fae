"""The pins catch plausible mistakes in the oracle.

Each case copies the C oracle source, plants one mistake (a dropped term, a
flipped sign or tie order, an off-by-one visibility rule, a wrong index or
exponent bias), builds the copy into a temporary library on the CPU, swaps it
in, and checks that at least one pin in test_oracle_pins.py fails.
"""
import ctypes
import os
import subprocess

import pytest

import test_oracle_pins as pins
from oracle import oracle as orc

MUTANTS = {
    "relu_dropped": ("s += Wt[h] * (dot > 0.0 ? dot : 0.0);", "s += Wt[h] * dot;"),
    "tie_to_higher_index": ("return (x->j < y->j) ? -1 : (x->j > y->j);",
                            "return (x->j > y->j) ? -1 : (x->j < y->j);"),
    "causal_strict": ("int64_t complete = (p + 1) / m;", "int64_t complete = p / m;"),
    "k_scale_dropped": ("double sc = k_scale ? (double)k_scale[j] : 1.0;\n        for (int i = 0; i < d; ++i)\n            K[j * d + i]",
                        "double sc = 1.0;\n        for (int i = 0; i < d; ++i)\n            K[j * d + i]"),
    "q_scale_wrong_row": ("q_scale[r * H + h]", "q_scale[h]"),
    "tail_short": ("*r = (expand && tail) ? (p + 1) - (*P) * m : 0;",
                   "*r = (expand && tail) ? p - (*P) * m : 0;"),
    "e4m3_bias": ("v = ldexp(8.0 + (double)f, e - 7 - 3);", "v = ldexp(8.0 + (double)f, e - 8 - 3);"),
    "weight_sign_lost": ("Wt[h] = (double)w[r * w_stride + h];", "Wt[h] = fabs((double)w[r * w_stride + h]);"),
    "operands_transposed": ("dot += Q[h * d + i] * Kj[i];", "dot += Q[i * H + h] * Kj[i];"),
    "pool_not_expanded": ("row[cnt++] = (int32_t)(cand[i].j * mexp + e);",
                          "row[cnt++] = (int32_t)(cand[i].j + e);"),
}

PIN_TESTS = [
    pins.test_we1_scores_and_rows,
    pins.test_we2_tie_rule,
    lambda: pins.test_all_zero_queries_every_key_ties(3),
    pins.test_we3_watch_lengths_and_width,
    pins.test_we4_pool_leak,
    pins.test_we5_csa_counts,
    pins.test_decode_e4m3_all_codes_match_torch,
    lambda: pins.test_scaled_configs_match_brute_force("c3_dsa_token"),
    lambda: pins.test_scaled_configs_match_brute_force("c2_glm_pooled"),
    pins.test_reduces_to_stable_argsort,
    pins.test_oracle_matches_brute_force_on_random_tiny_cases,
]


def _build_mutant(tmp_path, name):
    src = open(orc.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = os.path.join(tmp_path, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(tmp_path, f"lib{name}.so")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", path,
                           "-o", so, "-lm"])
    return so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name, monkeypatch):
    so = _build_mutant(str(tmp_path), name)
    good = orc._load()
    bad = ctypes.CDLL(so)
    for fn in ("oracle_select_rows", "oracle_pair_scores", "oracle_decode_bf16",
               "oracle_decode_e4m3", "oracle_output_width", "oracle_max_threads"):
        g, b = getattr(good, fn), getattr(bad, fn)
        b.restype, b.argtypes = g.restype, g.argtypes
    monkeypatch.setattr(orc, "_lib", bad)
    caught = []
    for pin in PIN_TESTS:
        try:
            pin()
        except (AssertionError, RuntimeError):
            caught.append(pin)
            break
    assert caught, f"no pin fails for mutant {name}"
