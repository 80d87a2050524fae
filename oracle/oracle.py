"""CPU oracle for the lightning-indexer step -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this module.  It shares no code with the HIP library
(``dsa_indexer_score_amd``) and neither imports the other; they meet only
through the seeded inputs of ``workloads``.

Pieces:
* ``select_rows`` / ``pair_scores``: the fp64 C oracle (indexer_oracle.c),
  naive score loops plus a full sort, see that file's header.
* ``select_rows_varlen``: packed documents, each document solved on its own
  rows and keys by the same oracle and mapped to global indices.
* ``output_width``, ``visible_keys``, ``tail_len``, ``expected_valid_len``:
  the visibility and slot arithmetic of GLM-5.3-Flash Module 06 "DSA &
  KPool" (section 2: 512 pools x 4 + 3 tail = 2,051 slots; section 3:
  pool-completion causality and the watch-length table).
* ``pair_overlap`` / ``overlap_stats``: the adjacent-pair statistic of
  "Adjacent-Query KV-Index Overlap in 256K DSA Training" (sections 1 and 3):
  non-overlapping pairs (q0,q1), (q2,q3), ...; exact set intersection of the
  sorted rows; overlap normalised by the valid top-k length of the rows
  (read as min(vA, vB)); Jaccard = shared / (vA + vB - shared).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "indexer_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

DTYPE_CODE = {"f32": 0, "bf16": 1, "fp8": 2}

_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (OpenMP threads over rows)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
                               SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(LIB)
        P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_select_rows.restype = I32
        lib.oracle_select_rows.argtypes = [P, P, P, I64, P, P, I32, I64, P, I64, I32, I32, I32,
                                           I32, I32, I32, I32, P, P, P, P, P, P, I32]
        lib.oracle_pair_scores.restype = I32
        lib.oracle_pair_scores.argtypes = [P, P, P, I64, P, P, I32, I64, I32, I32, I64, P, P,
                                           P, I32]
        lib.oracle_pair_bounds.restype = I32
        lib.oracle_pair_bounds.argtypes = lib.oracle_pair_scores.argtypes
        lib.oracle_decode_bf16.restype = D
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_e4m3.restype = D
        lib.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
        lib.oracle_output_width.restype = I32
        lib.oracle_output_width.argtypes = [I32, I32, I32, I32]
        lib.oracle_max_threads.restype = I32
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


# --------------------------------------------------------------------------
# Host-side arithmetic (GLM-5.3-Flash Module 06, sections 2 and 3).
# --------------------------------------------------------------------------
def output_width(topk: int, m: int, expand: bool, tail: bool) -> int:
    return topk + (m - 1 if (expand and tail) else 0)


def visible_keys(p: int, T: int, m: int, causal: bool) -> int:
    """Number of selectable keys for absolute position p: pools whose last
    token is at or before p (tokens when m = 1), capped at T."""
    if not causal:
        return T
    return min(T, (p + 1) // m)


def tail_len(p: int, T: int, m: int, causal: bool, expand: bool, tail: bool) -> int:
    if not (causal and expand and tail):
        return 0
    return (p + 1) - visible_keys(p, T, m, causal) * m


def expected_valid_len(p, T, m, topk, causal, expand, tail) -> int:
    P = visible_keys(p, T, m, causal)
    if expand:
        return min(topk // m, P) * m + tail_len(p, T, m, causal, expand, tail)
    return min(topk, P)


# --------------------------------------------------------------------------
# fp64 selection and scores.
# --------------------------------------------------------------------------
def _host(t):
    """torch tensor (any device) or ndarray -> contiguous host ndarray of raw bytes."""
    if t is None:
        return None
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().to("cpu").contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            if t.dtype == torch.float8_e4m3fn:
                return t.view(torch.uint8).numpy()
            return t.numpy()
    except ImportError:
        pass
    return np.ascontiguousarray(t)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _gather_rows(inp, rows):
    """Gather the q / q_scale / w rows of ``inp`` (an IndexerInputs) on its
    device, then copy only those to the host."""
    import torch
    rows_t = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=inp.q.device)
    q = _host(inp.q.index_select(0, rows_t))
    qs = None if inp.q_scale is None else _host(inp.q_scale.index_select(0, rows_t)).astype(np.float32)
    if inp.w.dim() == 1:
        w, wst = _host(inp.w).astype(np.float32), 0
    else:
        w, wst = _host(inp.w.index_select(0, rows_t)).astype(np.float32), inp.H
    return q, qs, np.ascontiguousarray(w), wst


def select_rows(inp, rows, nthreads: int = 0):
    """Run the oracle on rows ``rows`` (indices into inp.q) of an IndexerInputs.

    Returns a dict of numpy arrays: idx [n, W], valid_len [n], key_idx
    [n, Ksel], key_score [n, Ksel] (fp64), n_sel [n], tau [n].
    """
    rows = np.asarray(rows, dtype=np.int64)
    return _select(inp, rows, rows + inp.q_pos0, inp.k, inp.k_scale, inp.T, nthreads)


def _select(inp, rows, positions, k_t, ks_t, T, nthreads):
    """The C oracle on q rows ``rows`` of inp at the given absolute positions,
    against keys k_t [T, d] (scales ks_t)."""
    lib = _load()
    rows = np.asarray(rows, dtype=np.int64)
    n = rows.shape[0]
    q, qs, w, wst = _gather_rows(inp, rows)
    k = _host(k_t)
    ks = None if ks_t is None else _host(ks_t).astype(np.float32)
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    W = output_width(inp.topk, inp.m, inp.expand, inp.tail)
    Ksel = inp.topk // inp.m if inp.expand else inp.topk
    out = dict(
        idx=np.empty((n, W), np.int32), valid_len=np.empty(n, np.int32),
        key_idx=np.empty((n, Ksel), np.int32), key_score=np.empty((n, Ksel), np.float64),
        n_sel=np.empty(n, np.int32), tau=np.empty(n, np.float64),
    )
    rc = lib.oracle_select_rows(
        _ptr(q), _ptr(qs), _ptr(w), wst, _ptr(k), _ptr(ks), DTYPE_CODE[inp.dtype], n,
        _ptr(pos), T, inp.H, inp.d, inp.m, inp.topk, int(inp.causal), int(inp.expand),
        int(inp.tail), _ptr(out["idx"]), _ptr(out["valid_len"]), _ptr(out["key_idx"]),
        _ptr(out["key_score"]), _ptr(out["n_sel"]), _ptr(out["tau"]), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_select_rows failed with status {rc}")
    return out


def select_rows_varlen(inp, cu_q, cu_k, pos0=None, cu_tok=None, rows=None, nthreads: int = 0):
    """Packed documents -- GLM-5.3-Flash Module 06 "DSA & KPool", section 3
    and "Ship it": a pool never spans a document boundary and no document's
    tokens reach another document's selection.  Document i is the
    single-document problem on its own rows [cu_q[i], cu_q[i+1]), at
    positions pos0[i] + (row - cu_q[i]), against its own keys
    k[cu_k[i], cu_k[i+1]); its output entries are mapped to global indices:
    keys -> cu_k[i] + j, expanded positions (tail included) -> cu_tok[i] +
    position.  Rows outside every document are padding: all -1, length 0.
    Returns idx [n, W], valid_len [n] and key_idx [n, Ksel] (global keys,
    -1 past n_sel), n_sel [n]."""
    cu_q = np.asarray(cu_q, np.int64)
    cu_k = np.asarray(cu_k, np.int64)
    ndoc = cu_q.shape[0] - 1
    pos0 = np.zeros(ndoc, np.int64) if pos0 is None else np.asarray(pos0, np.int64)
    rows = np.arange(inp.S) if rows is None else np.asarray(rows, np.int64)
    W = output_width(inp.topk, inp.m, inp.expand, inp.tail)
    Ksel = inp.topk // inp.m if inp.expand else inp.topk
    n = rows.shape[0]
    out = dict(idx=np.full((n, W), -1, np.int32), valid_len=np.zeros(n, np.int32),
               key_idx=np.full((n, Ksel), -1, np.int64), n_sel=np.zeros(n, np.int32))
    for i in range(ndoc):
        at = np.nonzero((rows >= cu_q[i]) & (rows < cu_q[i + 1]))[0]
        if at.size == 0:
            continue
        k0, k1 = int(cu_k[i]), int(cu_k[i + 1])
        res = _select(inp, rows[at], pos0[i] + (rows[at] - cu_q[i]), inp.k[k0:k1],
                      None if inp.k_scale is None else inp.k_scale[k0:k1], k1 - k0, nthreads)
        base = int(cu_tok[i]) if inp.expand else k0
        idx = res["idx"].astype(np.int64)
        idx[idx >= 0] += base
        out["idx"][at] = idx.astype(np.int32)
        out["valid_len"][at] = res["valid_len"]
        for r, a in enumerate(at):
            ns = res["n_sel"][r]
            out["n_sel"][a] = ns
            out["key_idx"][a, :ns] = res["key_idx"][r, :ns] + k0
    return out


def pair_scores(inp, rows, keys, nthreads: int = 0, bounds: bool = False):
    """fp64 scores s*(rows[e], keys[e]) (rows index inp.q; keys index inp.k).
    With bounds=True, the condition sums sum_h |w_h| sum_i |q_hi k_i| instead."""
    lib = _load()
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.ascontiguousarray(np.asarray(keys, dtype=np.int64))
    uniq, inv = np.unique(rows, return_inverse=True)
    q, qs, w, wst = _gather_rows(inp, uniq)
    k = _host(inp.k)
    ks = None if inp.k_scale is None else _host(inp.k_scale).astype(np.float32)
    out = np.empty(rows.shape[0], np.float64)
    inv = np.ascontiguousarray(inv.astype(np.int64))
    fn = lib.oracle_pair_bounds if bounds else lib.oracle_pair_scores
    rc = fn(_ptr(q), _ptr(qs), _ptr(w), wst, _ptr(k), _ptr(ks),
                                DTYPE_CODE[inp.dtype], inp.T, inp.H, inp.d, rows.shape[0],
                                _ptr(inv), _ptr(keys), _ptr(out), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_pair_scores failed with status {rc}")
    return out


def decode_bf16(bits: int) -> float:
    return float(_load().oracle_decode_bf16(bits))


def decode_e4m3(bits: int) -> float:
    return float(_load().oracle_decode_e4m3(bits))


# --------------------------------------------------------------------------
# Adjacent-pair overlap diagnostic.
# --------------------------------------------------------------------------
def pair_overlap(idx: np.ndarray, valid_len: np.ndarray) -> np.ndarray:
    """shared[i] = |A_2i ∩ A_2i+1| for i < S // 2 (an odd last row is unpaired)."""
    idx = np.asarray(idx)
    vl = np.asarray(valid_len)
    npairs = idx.shape[0] // 2
    shared = np.empty(npairs, np.int32)
    for i in range(npairs):
        a = idx[2 * i, :vl[2 * i]]
        b = idx[2 * i + 1, :vl[2 * i + 1]]
        shared[i] = np.intersect1d(a, b, assume_unique=True).size
    return shared


def pair_regions(idx: np.ndarray, valid_len: np.ndarray):
    """Three-region split of each adjacent pair ("Adjacent-Query KV-Index
    Overlap in 256K DSA Training", sections 6.1 and 6.4): entries of both
    rows, only the left (row 2i), only the right (row 2i+1), each ascending
    and padded with -1 to the row width; counts [n, 3]."""
    idx = np.asarray(idx)
    vl = np.asarray(valid_len)
    n, W = idx.shape[0] // 2, idx.shape[1]
    out = [np.full((n, W), -1, np.int32) for _ in range(3)]
    counts = np.zeros((n, 3), np.int32)
    for i in range(n):
        a = idx[2 * i, :vl[2 * i]]
        b = idx[2 * i + 1, :vl[2 * i + 1]]
        parts = (np.intersect1d(a, b), np.setdiff1d(a, b), np.setdiff1d(b, a))
        for r, part in enumerate(parts):
            out[r][i, :part.size] = part
            counts[i, r] = part.size
    return out[0], out[1], out[2], counts


def overlap_stats(shared: np.ndarray, valid_len: np.ndarray) -> dict:
    """Page-1 table columns from per-pair shared counts and row valid lengths.
    Pairs with an empty row are excluded (their overlap is undefined)."""
    shared = np.asarray(shared, np.float64)
    vl = np.asarray(valid_len, np.float64)
    npairs = shared.shape[0]
    va, vb = vl[0:2 * npairs:2], vl[1:2 * npairs:2]
    ok = np.minimum(va, vb) > 0
    sh, va, vb = shared[ok], va[ok], vb[ok]
    if sh.size == 0:
        return dict(pairs=0, excluded=int(npairs))
    ov = sh / np.minimum(va, vb)
    jac = sh / (va + vb - sh)
    return dict(
        pairs=int(sh.size), excluded=int(npairs - sh.size),
        mean_overlap=float(ov.mean()), median_overlap=float(np.median(ov)),
        p90_overlap=float(np.percentile(ov, 90)), mean_jaccard=float(jac.mean()),
        mean_shared=float(sh.mean()), frac_ge_50=float((ov >= 0.5).mean()),
        frac_ge_75=float((ov >= 0.75).mean()), frac_ge_80=float((ov >= 0.8).mean()),
    )
