"""The DoSA certificate pins catch plausible mistakes in oracle/dosa.py.

Each case copies the module's source, plants one mistake (the activation
weight dropped from the negative-head priority, the majority boundary moved,
every omitted negative head aggregated, the joint bound's half or absolute
value lost, the projection coefficient left unclipped), loads the copy as a
separate module on the CPU and checks that at least one pin in
test_dosa_certificate.py fails against it.
"""
import importlib.util

import pytest

import test_dosa_certificate as pins
from oracle import dosa

MUTANTS = {
    "priority_without_activation": ("abs(w[h]) * norms[h] * min(p[h], 1 - p[h])",
                                    "abs(w[h]) * norms[h]"),
    "majority_strict": ("p[h] >= 0.5]", "p[h] > 0.5]"),
    "aggregate_every_omitted_negative": ("h not in kept and p[h] >= 0.5]", "h not in kept]"),
    "aggregate_without_weights": ("aA += abs(w[h]) * q[h]", "aA += q[h]"),
    "joint_without_half": ("E_joint = 0.5 * (", "E_joint = 1.0 * ("),
    "joint_signed_gram": ("np.sqrt(np.abs(U_res @ U_res.T).sum())",
                          "np.sqrt(max((U_res @ U_res.T).sum(), 0.0))"),
    "beta_unclipped": ("beta = max(q[h] @ q[j], 0.0) / (q[j] @ q[j])",
                       "beta = (q[h] @ q[j]) / (q[j] @ q[j])"),
    "residual_unweighted": ("U_res.append(w[h] * d_h)", "U_res.append(d_h)"),
}


def _load_mutant(tmp_path, name):
    src = open(dosa.__file__).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    path = tmp_path / f"dosa_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"dosa_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_pins_pass_on_the_oracle():
    for pin in pins.DOSA_PINS:
        pin(dosa)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_fails_on_mutant(tmp_path, name):
    mod = _load_mutant(tmp_path, name)
    failed = []
    for pin in pins.DOSA_PINS:
        try:
            pin(mod)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
    print(f"{name}: caught by {failed}")
