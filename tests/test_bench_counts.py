"""Host-side arithmetic of bench.py: the closed forms that turn a workload
into algorithmic work (visible pairs, pairs of the rows that are scored)
against brute force over the rows."""
import importlib.util
import os
import random

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def _visible(S, T, m, causal, q0):
    return [min(T, (q0 + t + 1) // m) if causal else T for t in range(S)]


def test_visible_and_scored_pairs_match_brute_force():
    rng = random.Random(5)
    for _ in range(2000):
        S, T = rng.randint(0, 300), rng.randint(0, 200)
        m, causal = rng.choice([1, 2, 4, 8]), rng.random() < 0.8
        ksel, q0 = rng.randint(1, 120), rng.randint(0, 400)
        P = _visible(S, T, m, causal, q0)
        assert bench.visible_pairs(S, T, m, causal, q0) == sum(P)
        assert bench.scored_pairs(S, T, m, causal, ksel, q0) == sum(p for p in P if p > ksel)


def test_scored_pairs_at_the_csa_prefill_shape():
    """S = 262,144 rows over 65,536 pools of 4, Ksel = 2048: the rows before
    position 8195 see at most 2048 pools and are not scored (0.1 % of the
    visible pairs)."""
    vis = bench.visible_pairs(262144, 65536, 4, True)
    sc = bench.scored_pairs(262144, 65536, 4, True, 2048)
    assert vis - sc == sum(min(65536, (t + 1) // 4) for t in range(8195))
    assert 0.998 < sc / vis < 0.9991


def test_gemm_context_reports_both_operand_kinds(monkeypatch):
    """The vendor-GEMM reference figure: n^3 matmuls timed on normal
    operands and on zeros, each as TFLOP/s (2 n^3 flop per call) and as a
    fraction of the bf16 dense peak.  Timed here on the CPU with a clock in
    place of the device events (the arithmetic, not the GPU)."""
    import time
    import torch

    class _Event:
        def __init__(self, enable_timing=True):
            self.t = 0.0

        def record(self, *args):
            self.t = time.perf_counter()

        def elapsed_time(self, other):
            return (other.t - self.t) * 1e3

    monkeypatch.setattr(torch.cuda, "Event", _Event)
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a: None)
    monkeypatch.setattr(torch.cuda, "empty_cache", lambda *a: None)
    ctx = bench.gemm_context("cpu", n=128, reps=2)
    assert ctx["shape"] == "128x128x128"
    for kind in ("random_normal", "zeros"):
        tf = ctx[f"{kind}_tflops"]
        assert tf > 0
        assert abs(ctx[f"{kind}_frac_of_bf16_peak"] - tf / bench.PEAK_TFLOPS["bf16"]) < 1e-12
