"""MI355X-native lightning indexer (DSA / CSA): scores, streaming top-k and
the adjacent-pair overlap diagnostic, all computed by HIP kernels for gfx950
behind the C ABI of include/dsa_indexer.h.

This module only marshals arguments: it checks tensor dtypes, shapes and
devices, allocates outputs and the workspace through PyTorch, and passes raw
pointers plus the current HIP stream to the library.  Nothing here computes
any part of the indexer, and there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import (IDX_BF16, IDX_EXPAND, IDX_F32, IDX_FP8_E4M3, IDX_FP8_MFMA,  # noqa: F401
                   IDX_SCREEN, IDX_TAIL)

__all__ = ["Indexer", "score_topk", "output_width", "pair_overlap", "overlap_summary",
           "library_path"]

_DTYPE_CODE = {torch.float32: IDX_F32, torch.bfloat16: IDX_BF16,
               torch.float8_e4m3fn: IDX_FP8_E4M3}


def library_path() -> str:
    _lib.load()
    return _lib.LIB_PATH


def _flags(expand: bool, tail: bool, screen: bool = False, fp8_mfma: bool = False) -> int:
    return (IDX_EXPAND if expand else 0) | (IDX_TAIL if tail else 0) | \
        (IDX_SCREEN if screen else 0) | (IDX_FP8_MFMA if fp8_mfma else 0)


def output_width(topk: int, m: int = 1, expand: bool = False, tail: bool = False) -> int:
    W = ctypes.c_int(0)
    _lib.check(_lib.load().indexer_output_width(int(topk), int(m), _flags(expand, tail),
                                                ctypes.byref(W)), "indexer_output_width")
    return W.value


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class Indexer:
    """A library handle: element dtype, output mode, rows per streaming
    launch (0: as many as 4 GiB of candidate buffers hold), the row count at
    or below which the few-query path runs (0: the library's default,
    negative: never), DoSA certificate screening of the streaming path
    (screen=True; used when 33 <= H <= 64) and, for e4m3 inputs, the
    contraction on the fp8 MFMA (fp8_mfma=True; d = 64 or 128, unscreened)."""

    def __init__(self, dtype: torch.dtype, *, expand: bool = False, tail: bool = False,
                 query_chunk: int = 0, few_query_rows: int = 0, screen: bool = False,
                 fp8_mfma: bool = False, device=None):
        if dtype not in _DTYPE_CODE:
            raise TypeError(f"unsupported dtype {dtype}")
        dev = torch.device("cuda") if device is None else torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.dtype, self.expand, self.tail = dtype, bool(expand), bool(tail)
        self.query_chunk = int(query_chunk or 0)
        self.few_query_rows = int(few_query_rows or 0)
        self.screen = bool(screen)
        self.fp8_mfma = bool(fp8_mfma)
        cfg = _lib.IndexerConfig(_DTYPE_CODE[dtype], _flags(expand, tail, screen, fp8_mfma),
                                 self.query_chunk, self.few_query_rows)
        h = ctypes.c_void_p()
        lib = _lib.load()
        _lib.check(lib.indexer_create(ctypes.byref(cfg), self.device.index or 0, ctypes.byref(h)),
                   "indexer_create")
        self._h = h
        self._lib = lib

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.indexer_destroy(h)
            self._h = None

    def _inputs(self, q, w, k, q_scale, k_scale):
        """Check q, w, k and the fp8 scales; returns (S, H, d, T, w_stride)."""
        if q.dim() != 3 or k.dim() != 2:
            raise ValueError("q must be [S, H, d] and k [T, d]")
        S, H, d = q.shape
        T = k.shape[0]
        if q.dtype != self.dtype or k.dtype != self.dtype:
            raise TypeError(f"q and k must be {self.dtype}")
        if k.shape[1] != d:
            raise ValueError("q and k disagree on d")
        for name, t in (("q", q), ("k", k), ("w", w), ("q_scale", q_scale), ("k_scale", k_scale)):
            if t is not None and (t.device != self.device or not t.is_contiguous()):
                raise ValueError(f"{name} must be contiguous on {self.device}")
        if w.dtype != torch.float32:
            raise TypeError("w must be float32")
        if w.dim() == 1 and w.shape[0] == H:
            w_stride = 0
        elif w.dim() == 2 and tuple(w.shape) == (S, H):
            w_stride = H
        else:
            raise ValueError("w must be [H] or [S, H]")
        if self.dtype == torch.float8_e4m3fn:
            if q_scale is None or k_scale is None:
                raise ValueError("fp8 needs q_scale [S,H] and k_scale [T]")
            if tuple(q_scale.shape) != (S, H) or tuple(k_scale.shape) != (T,) or \
                    q_scale.dtype != torch.float32 or k_scale.dtype != torch.float32:
                raise ValueError("q_scale must be float32 [S,H], k_scale float32 [T]")
        elif q_scale is not None or k_scale is not None:
            raise ValueError("q_scale / k_scale are for fp8 only")
        return S, H, d, T, w_stride

    def _outputs(self, S, W, with_scores, out):
        """Allocate (idx, valid_len, sel) or check the caller's: contiguous,
        on this device, int32 [S, W] / int32 [S] / float32 [S, W] or None."""
        if out is None:
            idx = torch.empty((S, W), dtype=torch.int32, device=self.device)
            valid_len = torch.empty((S,), dtype=torch.int32, device=self.device)
            sel = torch.empty((S, W), dtype=torch.float32, device=self.device) \
                if with_scores else None
            return idx, valid_len, sel
        idx, valid_len, sel = out
        for name, t, dt, shape in (("idx", idx, torch.int32, (S, W)),
                                   ("valid_len", valid_len, torch.int32, (S,)),
                                   ("sel_score", sel, torch.float32, (S, W))):
            if t is None and name == "sel_score":
                continue
            if t is None or t.dtype != dt or tuple(t.shape) != shape or \
                    t.device != self.device or not t.is_contiguous():
                raise ValueError(f"out {name} must be a contiguous {dt} tensor of shape "
                                 f"{shape} on {self.device}")
        if with_scores and sel is None:
            raise ValueError("with_scores needs a sel_score tensor in out")
        return idx, valid_len, sel

    def _workspace(self, nbytes, workspace):
        if workspace is None:
            return torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=self.device)
        if workspace.dtype != torch.uint8 or workspace.dim() != 1 or \
                not workspace.is_contiguous() or workspace.device != self.device or \
                workspace.numel() < nbytes:
            raise ValueError(f"workspace must be a contiguous uint8 tensor of at least {nbytes} "
                             f"bytes on {self.device}")
        return workspace

    def workspace_bytes(self, S: int, T: int, H: int, d: int, m: int, topk: int) -> int:
        n = ctypes.c_size_t(0)
        _lib.check(self._lib.indexer_workspace_bytes(self._h, S, T, H, d, m, topk, ctypes.byref(n)),
                   "indexer_workspace_bytes")
        return n.value

    def score_topk(self, q, w, k, *, m: int = 1, topk: int, causal: bool = True,
                   q_scale=None, k_scale=None, q_pos0: int = 0, with_scores: bool = False,
                   workspace: Optional[torch.Tensor] = None, out=None, witness=None):
        """q [S,H,d], w [S,H] or [H] (fp32), k [T,d] -> (idx [S,W] int32,
        valid_len [S] int32[, sel_score [S,W] fp32]) on q's device.  out =
        (idx, valid_len, sel_score or None) writes into the caller's tensors.
        witness (int32 [S, n] on q's device, e.g. the rows' idx of an earlier
        step) goes through indexer_score_topk_witness."""
        S, H, d, T, w_stride = self._inputs(q, w, k, q_scale, k_scale)
        W = output_width(topk, m, self.expand, self.tail)
        idx, valid_len, sel = self._outputs(S, W, with_scores, out)
        workspace = self._workspace(self.workspace_bytes(S, T, H, d, m, topk), workspace)
        common = (self._h, _ptr(q), _ptr(q_scale), _ptr(w), w_stride, _ptr(k), _ptr(k_scale), S,
                  T, H, d, m, topk, int(bool(causal)), int(q_pos0))
        tail = (_ptr(idx), _ptr(valid_len), _ptr(sel), _ptr(workspace),
                workspace.numel() * workspace.element_size(), _stream(self.device))
        if witness is None:
            rc = self._lib.indexer_score_topk(*common, *tail)
            _lib.check(rc, "indexer_score_topk")
        else:
            if (witness.dim() != 2 or witness.shape[0] != S or witness.dtype != torch.int32
                    or witness.device != self.device or not witness.is_contiguous()):
                raise ValueError("witness must be a contiguous int32 [S, n] tensor on the device")
            n = witness.shape[1]
            rc = self._lib.indexer_score_topk_witness(*common, _ptr(witness), n, n, *tail)
            _lib.check(rc, "indexer_score_topk_witness")
        return (idx, valid_len, sel) if with_scores else (idx, valid_len)


    def score_topk_noalloc(self, q, w, k, *, m: int = 1, topk: int, causal: bool = True,
                           q_scale=None, k_scale=None, q_pos0: int = 0,
                           with_scores: bool = False, out=None):
        """score_topk through indexer_score_topk_noalloc: no workspace, the
        library's static scratch instead (same results).  With out given,
        nothing is allocated here either."""
        S, H, d, T, w_stride = self._inputs(q, w, k, q_scale, k_scale)
        W = output_width(topk, m, self.expand, self.tail)
        idx, valid_len, sel = self._outputs(S, W, with_scores, out)
        rc = self._lib.indexer_score_topk_noalloc(
            self._h, _ptr(q), _ptr(q_scale), _ptr(w), w_stride, _ptr(k), _ptr(k_scale), S, T, H,
            d, m, topk, int(bool(causal)), int(q_pos0), _ptr(idx), _ptr(valid_len), _ptr(sel),
            _stream(self.device))
        _lib.check(rc, "indexer_score_topk_noalloc")
        return (idx, valid_len, sel) if with_scores else (idx, valid_len)

    def workspace_bytes_varlen(self, S: int, T: int, H: int, d: int, m: int, topk: int,
                               ndoc: int, max_doc_keys: int = 0) -> int:
        n = ctypes.c_size_t(0)
        _lib.check(self._lib.indexer_workspace_bytes_varlen(self._h, S, T, H, d, m, topk, ndoc,
                                                            max_doc_keys, ctypes.byref(n)),
                   "indexer_workspace_bytes_varlen")
        return n.value

    def score_topk_varlen(self, q, w, k, cu_q, cu_k, *, m: int = 1, topk: int,
                          causal: bool = True, pos0=None, cu_tok=None, q_scale=None,
                          k_scale=None, max_doc_keys: int = 0, with_scores: bool = False,
                          workspace: Optional[torch.Tensor] = None, out=None):
        """Packed documents: rows [cu_q[i], cu_q[i+1]) see keys [cu_k[i], cu_k[i+1])
        (int32 device tensors of ndoc + 1 entries); pos0 (int64 [ndoc]) is each
        document's first-row position, cu_tok (int32 [ndoc], expand mode) its
        token offset; max_doc_keys (host int, 0 = unknown) bounds every
        document's key count and sizes the few-query path's dense rows.
        Returns (idx, valid_len[, sel_score])."""
        S, H, d, T, w_stride = self._inputs(q, w, k, q_scale, k_scale)
        ndoc = cu_q.numel() - 1
        if ndoc < 0 or cu_k.numel() != ndoc + 1:
            raise ValueError("cu_q and cu_k must both have ndoc + 1 entries")
        for name, t, dt in (("cu_q", cu_q, torch.int32), ("cu_k", cu_k, torch.int32),
                            ("pos0", pos0, torch.int64), ("cu_tok", cu_tok, torch.int32)):
            if t is None:
                continue
            if t.dtype != dt or t.device != self.device or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {dt} tensor on {self.device}")
            if name in ("pos0", "cu_tok") and t.numel() != ndoc:
                raise ValueError(f"{name} must have ndoc entries")
        W = output_width(topk, m, self.expand, self.tail)
        idx, valid_len, sel = self._outputs(S, W, with_scores, out)
        workspace = self._workspace(
            self.workspace_bytes_varlen(S, T, H, d, m, topk, ndoc, max_doc_keys), workspace)
        rc = self._lib.indexer_score_topk_varlen(
            self._h, _ptr(q), _ptr(q_scale), _ptr(w), w_stride, _ptr(k), _ptr(k_scale), S, T, H,
            d, m, topk, int(bool(causal)), _ptr(cu_q), _ptr(cu_k), _ptr(pos0), _ptr(cu_tok), ndoc,
            max_doc_keys, _ptr(idx), _ptr(valid_len), _ptr(sel), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(self.device))
        _lib.check(rc, "indexer_score_topk_varlen")
        return (idx, valid_len, sel) if with_scores else (idx, valid_len)


_HANDLES = {}


def _handle(dtype, expand, tail, query_chunk, few_query_rows, device, screen=False,
            fp8_mfma=False) -> Indexer:
    key = (dtype, bool(expand), bool(tail), int(query_chunk or 0), int(few_query_rows or 0),
           bool(screen), bool(fp8_mfma), str(torch.device(device)))
    h = _HANDLES.get(key)
    if h is None:
        h = _HANDLES[key] = Indexer(dtype, expand=expand, tail=tail, query_chunk=query_chunk,
                                    few_query_rows=few_query_rows, screen=screen,
                                    fp8_mfma=fp8_mfma, device=device)
    return h


def score_topk(q, w, k, *, m: int = 1, topk: int, causal: bool = True, expand: bool = False,
               tail: bool = False, q_scale=None, k_scale=None, q_pos0: int = 0,
               query_chunk: int = 0, few_query_rows: int = 0, screen: bool = False,
               fp8_mfma: bool = False, with_scores: bool = False, workspace=None):
    """One indexer step; see Indexer.score_topk."""
    return _handle(q.dtype, expand, tail, query_chunk, few_query_rows, q.device,
                   screen, fp8_mfma).score_topk(
        q, w, k, m=m, topk=topk, causal=causal, q_scale=q_scale, k_scale=k_scale,
        q_pos0=q_pos0, with_scores=with_scores, workspace=workspace)


def screen_certificates(q: torch.Tensor, w: torch.Tensor, q_scale=None, k=None, *, m: int = 1,
                        causal: bool = True, q_pos0: int = 0):
    """The DoSA certificates the screened path builds for each row of q
    [S, H, d] (33 <= H <= 64), with seeds from the keys k [T, d] (none when
    k is None): (perm int32 [S, 64], weights [S, 64], bound_weights [S, 32],
    knorm_coef [S], aggregate [S, d], activations int32 [S, 64]) on q's
    device; see indexer_screen_certificates.  Rows without an aggregate
    leave their aggregate row zero."""
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [S, H, d] tensor")
    S, H, d = q.shape
    if w.dtype != torch.float32 or not w.is_contiguous() or w.device != q.device:
        raise ValueError("w must be contiguous float32 on q's device")
    if w.dim() == 1 and w.shape[0] == H:
        w_stride = 0
    elif w.dim() == 2 and tuple(w.shape) == (S, H):
        w_stride = H
    else:
        raise ValueError("w must be [H] or [S, H]")
    if (q.dtype == torch.float8_e4m3fn) != (q_scale is not None):
        raise ValueError("q_scale [S, H] float32 is required exactly for fp8")
    if q_scale is not None and (tuple(q_scale.shape) != (S, H) or
                                q_scale.dtype != torch.float32 or
                                not q_scale.is_contiguous() or q_scale.device != q.device):
        raise ValueError("q_scale must be contiguous float32 [S, H] on q's device")
    T = 0
    if k is not None:
        if (k.dim() != 2 or k.shape[1] != d or k.dtype != q.dtype or not k.is_contiguous()
                or k.device != q.device):
            raise ValueError("k must be a contiguous [T, d] tensor of q's dtype and device")
        T = k.shape[0]
    h = _handle(q.dtype, False, False, 0, 0, q.device)
    dev = h.device
    perm = torch.empty((S, 64), dtype=torch.int32, device=dev)
    wv = torch.empty((S, 64), dtype=torch.float32, device=dev)
    wt = torch.empty((S, 32), dtype=torch.float32, device=dev)
    e = torch.empty((S,), dtype=torch.float32, device=dev)
    agg = torch.zeros((S, d), dtype=torch.float32, device=dev)
    act = torch.empty((S, 64), dtype=torch.int32, device=dev)
    _lib.check(h._lib.indexer_screen_certificates(
        h._h, _ptr(q), _ptr(q_scale), _ptr(w), w_stride, S, H, d, _ptr(k), T, int(m),
        int(bool(causal)), int(q_pos0), _ptr(perm), _ptr(wv), _ptr(wt), _ptr(e), _ptr(agg),
        _ptr(act), _stream(dev)), "indexer_screen_certificates")
    return perm, wv, wt, e, agg, act


def pair_overlap(idx: torch.Tensor, valid_len: torch.Tensor) -> torch.Tensor:
    """shared[i] = |row 2i ∩ row 2i+1| (device int32 [S//2])."""
    if idx.dim() != 2 or idx.dtype != torch.int32 or valid_len.dtype != torch.int32:
        raise TypeError("idx must be int32 [S, W] and valid_len int32 [S]")
    if not (idx.is_cuda and idx.is_contiguous() and valid_len.is_cuda):
        raise ValueError("idx / valid_len must be contiguous device tensors")
    S, W = idx.shape
    shared = torch.empty((S // 2,), dtype=torch.int32, device=idx.device)
    lib = _lib.load()
    _lib.check(lib.indexer_pair_overlap(_ptr(idx), _ptr(valid_len), S, W, _ptr(shared),
                                        _stream(idx.device)), "indexer_pair_overlap")
    return shared


def pair_regions(idx: torch.Tensor, valid_len: torch.Tensor):
    """Per adjacent pair: (shared, left_only, right_only) rows [S//2, W]
    (ascending, then -1) and counts [S//2, 3], all device int32."""
    if idx.dim() != 2 or idx.dtype != torch.int32 or valid_len.dtype != torch.int32:
        raise TypeError("idx must be int32 [S, W] and valid_len int32 [S]")
    if not (idx.is_cuda and idx.is_contiguous() and valid_len.is_cuda):
        raise ValueError("idx / valid_len must be contiguous device tensors")
    S, W = idx.shape
    n = S // 2
    shared, left, right = (torch.empty((n, W), dtype=torch.int32, device=idx.device)
                           for _ in range(3))
    counts = torch.empty((n, 3), dtype=torch.int32, device=idx.device)
    lib = _lib.load()
    _lib.check(lib.indexer_pair_regions(_ptr(idx), _ptr(valid_len), S, W, _ptr(shared),
                                        _ptr(left), _ptr(right), _ptr(counts),
                                        _stream(idx.device)), "indexer_pair_regions")
    return shared, left, right, counts


def overlap_summary(shared: torch.Tensor, valid_len: torch.Tensor) -> dict:
    """Page-1 style statistics (host computation over host copies)."""
    sh = shared.detach().to("cpu", torch.int32).contiguous()
    vl = valid_len.detach().to("cpu", torch.int32).contiguous()
    st = _lib.OverlapStats()
    lib = _lib.load()
    _lib.check(lib.indexer_overlap_summary(_ptr(sh), _ptr(vl), vl.numel(), ctypes.byref(st)),
               "indexer_overlap_summary")
    return {name: getattr(st, name) for name, _ in _lib.OverlapStats._fields_}
