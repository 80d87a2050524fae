"""Seeded synthetic workloads for the lightning-indexer step.

Each workload reproduces the shapes and value distributions of one of the
five benchmark configurations (tiny integer-exact, GLM-style pooled, DSA
token-level, CSA 256K, CSA 1M).  The recipe, per tensor:

* integer config: q, k uniform on {-3..3} held in fp32; w drawn per
  (query, head) from {-1, -0.5, 0.5, 1}.
* float configs: q, k ~ N(0, 1/d); w ~ N(0, 1) drawn once per head and
  broadcast to every query (``w`` has shape [H]).
* GLM-style pooled keys: token keys ~ N(0, 1/d) rounded to bf16, pooled
  key = fp32 mean of m consecutive bf16 token keys, rounded once to bf16.
* AR(1) queries (DSA token-level and 1M CSA): along the sequence, for every
  (head, channel): q_0 = e_0, q_t = rho q_{t-1} + sqrt(1 - rho^2) e_t with
  e ~ N(0, 1/d), rho = 0.9, so adjacent queries are correlated.
* fp8: OCP e4m3 (float8_e4m3fn) with an fp32 scale per row of d values
  (per (query, head) for q, per key for k): scale = amax / 448 (1 for an
  all-zero row), code = RNE(clamp(x / scale, -448, 448)).
* bf16: round-to-nearest-even from fp32 (torch's conversion).

Seeds: base 0x5EED0000 + config number; q, k and w use independent
generators (base + 1, base + 2, base + 3).

No arithmetic of the method lives here: this module never scores, masks or
selects anything.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

# --------------------------------------------------------------------------
# The five workloads.  ``T`` is derived from ``S`` when a config is scaled:
# token-level configs keep T = S, pooled / compressed configs keep T = S / m.
# --------------------------------------------------------------------------
CONFIGS = {
    "c1_tiny_int": dict(
        number=1, S=1024, T=1024, m=1, H=4, d=32, topk=64, causal=True,
        expand=False, tail=False, dtype="f32", qdist="int", kdist="int",
        wdist="int_per_row", t_rule="same", query_chunk=None,
    ),
    "c2_glm_pooled": dict(
        number=2, S=32768, T=8192, m=4, H=32, d=128, topk=2048, causal=True,
        expand=True, tail=True, dtype="bf16", qdist="normal", kdist="pooled",
        wdist="normal_bcast", t_rule="div_m", query_chunk=None,
    ),
    "c3_dsa_token": dict(
        number=3, S=131072, T=131072, m=1, H=64, d=128, topk=2048, causal=True,
        expand=False, tail=False, dtype="fp8", qdist="ar1", kdist="normal",
        wdist="normal_bcast", t_rule="same", query_chunk=32768,
    ),
    "c4_csa_256k": dict(
        number=4, S=262144, T=65536, m=4, H=64, d=128, topk=2048, causal=True,
        expand=False, tail=False, dtype="bf16", qdist="normal", kdist="normal",
        wdist="normal_bcast", t_rule="div_m", query_chunk=16384,
    ),
    "c5_csa_1m": dict(
        number=5, S=1048576, T=262144, m=4, H=64, d=128, topk=2048, causal=True,
        expand=False, tail=False, dtype="fp8", qdist="ar1", kdist="normal",
        wdist="normal_bcast", t_rule="div_m", query_chunk=32768,
    ),
}

AR1_RHO = 0.9
E4M3_MAX = 448.0


def config_names():
    return list(CONFIGS)


@dataclass
class IndexerInputs:
    """One seeded indexer problem, laid out as the C ABI consumes it.

    q        [S, H, d]  float32 / bfloat16 / float8_e4m3fn
    q_scale  [S, H]     float32 (fp8 only, else None)
    w        [S, H] or [H] float32 ([H] means one row broadcast to all queries)
    k        [T, d]     same dtype as q
    k_scale  [T]        float32 (fp8 only, else None)
    """

    name: str
    S: int
    T: int
    H: int
    d: int
    m: int
    topk: int
    causal: bool
    expand: bool
    tail: bool
    dtype: str
    q: torch.Tensor
    q_scale: Optional[torch.Tensor]
    w: torch.Tensor
    k: torch.Tensor
    k_scale: Optional[torch.Tensor]
    q_pos0: int = 0
    query_chunk: Optional[int] = None
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def w_stride_s(self) -> int:
        return 0 if self.w.dim() == 1 else self.H

    def to(self, device) -> "IndexerInputs":
        mv = lambda t: None if t is None else t.to(device)  # noqa: E731
        return replace(self, q=mv(self.q), q_scale=mv(self.q_scale), w=mv(self.w),
                       k=mv(self.k), k_scale=mv(self.k_scale))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size()
                   for t in (self.q, self.q_scale, self.w, self.k, self.k_scale)
                   if t is not None)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def quant_e4m3_rows(x: torch.Tensor):
    """fp32 [..., d] -> (float8_e4m3fn [..., d], fp32 scale [...])."""
    x = x.float()
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return y, scale.contiguous()


def _normal(shape, d, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) / math.sqrt(d)


def _ar1_chunks(S, H, d, rho, g, device, chunk_rows):
    """Yield fp32 [n, H, d] chunks of the AR(1) sequence, in order."""
    L = 64
    chunk_rows = max(L, (chunk_rows // L) * L)
    c = math.sqrt(1.0 - rho * rho)
    i = torch.arange(L, device=device, dtype=torch.float32)
    expo = (i[:, None] - i[None, :]).clamp(min=0)
    A = torch.where(i[:, None] >= i[None, :], rho ** expo, torch.zeros_like(expo))
    carry_pow = (rho ** (i + 1)).unsqueeze(-1)  # [L, 1]
    hd = H * d
    prev = None
    for r0 in range(0, S, chunk_rows):
        n = min(chunk_rows, S - r0)
        eps = _normal((n, hd), d, g, device)
        innov = eps * c
        if r0 == 0:
            innov[0] = eps[0]
        nb = (n + L - 1) // L
        if nb * L != n:
            innov = torch.cat([innov, innov.new_zeros(nb * L - n, hd)], 0)
        Z = torch.matmul(A, innov.view(nb, L, hd).contiguous())  # [nb, L, hd]
        out = torch.empty_like(Z)
        for b in range(nb):
            if prev is None:
                out[b] = Z[b]
            else:
                out[b] = Z[b] + carry_pow * prev
            prev = out[b, L - 1]
        yield out.view(nb * L, hd)[:n].view(n, H, d)


def generate(name: str, *, S: Optional[int] = None, T: Optional[int] = None,
             topk: Optional[int] = None, seed: Optional[int] = None,
             device="cpu", gen_chunk_rows: int = 16384, **overrides) -> IndexerInputs:
    """Draw one workload.  ``S`` (and optionally ``T``/``topk``) scale it down
    while keeping the config's dtype, distributions and mode."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    S = cfg["S"] if S is None else int(S)
    if T is None:
        if S == cfg["S"]:
            T = cfg["T"]
        elif cfg["t_rule"] == "same":
            T = S
        else:
            T = S // cfg["m"]
    topk = cfg["topk"] if topk is None else int(topk)
    H, d, m = cfg["H"], cfg["d"], cfg["m"]
    base = 0x5EED0000 + cfg["number"] if seed is None else int(seed)
    device = torch.device(device)
    gq, gk, gw = _gen(device, base + 1), _gen(device, base + 2), _gen(device, base + 3)

    dtype = cfg["dtype"]
    q_scale = k_scale = None

    # ---- queries
    if cfg["qdist"] == "int":
        q = torch.randint(-3, 4, (S, H, d), generator=gq, device=device).float()
    elif cfg["qdist"] == "normal":
        q = _normal((S, H, d), d, gq, device)
    elif cfg["qdist"] == "ar1":
        q = None
    else:
        raise ValueError(cfg["qdist"])

    if dtype == "fp8":
        q8 = torch.empty((S, H, d), dtype=torch.float8_e4m3fn, device=device)
        q_scale = torch.empty((S, H), dtype=torch.float32, device=device)
        if q is None:
            r0 = 0
            for chunk in _ar1_chunks(S, H, d, cfg.get("rho", AR1_RHO), gq, device, gen_chunk_rows):
                n = chunk.shape[0]
                q8[r0:r0 + n], q_scale[r0:r0 + n] = quant_e4m3_rows(chunk)
                r0 += n
        else:
            for r0 in range(0, S, gen_chunk_rows):
                q8[r0:r0 + gen_chunk_rows], q_scale[r0:r0 + gen_chunk_rows] = \
                    quant_e4m3_rows(q[r0:r0 + gen_chunk_rows])
        q = q8
    else:
        if q is None:
            q = torch.cat(list(_ar1_chunks(S, H, d, cfg.get("rho", AR1_RHO), gq, device, gen_chunk_rows)), 0)
        if dtype == "bf16":
            q = q.to(torch.bfloat16)
        elif dtype != "f32":
            raise ValueError(dtype)

    # ---- keys
    if cfg["kdist"] == "int":
        k = torch.randint(-3, 4, (T, d), generator=gk, device=device).float()
    elif cfg["kdist"] == "normal":
        k = _normal((T, d), d, gk, device)
    elif cfg["kdist"] == "pooled":
        tok = _normal((T * m, d), d, gk, device).to(torch.bfloat16).float()
        k = tok.view(T, m, d).mean(dim=1)
    else:
        raise ValueError(cfg["kdist"])
    if dtype == "fp8":
        k, k_scale = quant_e4m3_rows(k)
    elif dtype == "bf16":
        k = k.to(torch.bfloat16)

    # ---- head weights
    if cfg["wdist"] == "int_per_row":
        vals = torch.tensor([-1.0, -0.5, 0.5, 1.0], device=device)
        w = vals[torch.randint(0, 4, (S, H), generator=gw, device=device)]
    elif cfg["wdist"] == "normal_bcast":
        w = torch.randn((H,), generator=gw, device=device, dtype=torch.float32)
    elif cfg["wdist"] == "lognormal_bcast":
        # signed weights whose magnitudes spread over decades (a few dominant
        # heads): a synthetic stand-in for trained head weights, where
        # certificate screening prunes (override of any config)
        z = torch.randn((2, H), generator=gw, device=device, dtype=torch.float32)
        w = z[0] * torch.exp(1.5 * z[1])
    else:
        raise ValueError(cfg["wdist"])

    return IndexerInputs(
        name=name, S=S, T=T, H=H, d=d, m=m, topk=topk, causal=cfg["causal"],
        expand=cfg["expand"], tail=cfg["tail"], dtype=dtype,
        q=q.contiguous(), q_scale=q_scale, w=w.contiguous(), k=k.contiguous(),
        k_scale=k_scale, q_pos0=0, query_chunk=cfg["query_chunk"], seed=base,
        meta=dict(qdist=cfg["qdist"], kdist=cfg["kdist"], wdist=cfg["wdist"]),
    )


def custom(*, q, k, w, m=1, topk, causal=True, expand=False, tail=False,
           q_scale=None, k_scale=None, q_pos0=0, name="custom") -> IndexerInputs:
    """Wrap hand-built tensors (worked examples, degenerate cases)."""
    S, H, d = q.shape
    T = k.shape[0]
    if q.dtype == torch.float8_e4m3fn:
        dtype = "fp8"
    elif q.dtype == torch.bfloat16:
        dtype = "bf16"
    else:
        dtype = "f32"
    return IndexerInputs(name=name, S=S, T=T, H=H, d=d, m=m, topk=topk, causal=causal,
                         expand=expand, tail=tail, dtype=dtype, q=q.contiguous(),
                         q_scale=q_scale, w=w.contiguous(), k=k.contiguous(),
                         k_scale=k_scale, q_pos0=q_pos0)
