"""ctypes view of libdsa_indexer.so (the C ABI of include/dsa_indexer.h)."""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa_indexer.so")

IDX_F32, IDX_BF16, IDX_FP8_E4M3 = 0, 1, 2
IDX_EXPAND, IDX_TAIL, IDX_SCREEN, IDX_FP8_MFMA = 1, 2, 4, 8
IDX_OK, IDX_EINVAL, IDX_EUNSUPPORTED, IDX_EWORKSPACE, IDX_EHIP = 0, -1, -2, -3, -4


class IndexerConfig(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("flags", ctypes.c_int), ("query_chunk", ctypes.c_int64),
                ("few_query_rows", ctypes.c_int64)]


class OverlapStats(ctypes.Structure):
    _fields_ = [("pairs", ctypes.c_int64), ("excluded", ctypes.c_int64),
                ("mean_overlap", ctypes.c_double), ("median_overlap", ctypes.c_double),
                ("p90_overlap", ctypes.c_double), ("mean_jaccard", ctypes.c_double),
                ("mean_shared", ctypes.c_double), ("frac_ge_50", ctypes.c_double),
                ("frac_ge_75", ctypes.c_double), ("frac_ge_80", ctypes.c_double)]


# name -> (restype, argtypes); mirrors include/dsa_indexer.h
_P, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "indexer_create": (_I, [ctypes.POINTER(IndexerConfig), _I, ctypes.POINTER(_P)]),
    "indexer_destroy": (_I, [_P]),
    "indexer_output_width": (_I, [_I, _I, _I, ctypes.POINTER(_I)]),
    "indexer_workspace_bytes": (_I, [_P, _I64, _I64, _I, _I, _I, _I, ctypes.POINTER(_SZ)]),
    "indexer_score_topk": (_I, [_P, _P, _P, _P, _I64, _P, _P, _I64, _I64, _I, _I, _I, _I, _I,
                                _I64, _P, _P, _P, _P, _SZ, _P]),
    "indexer_score_topk_noalloc": (_I, [_P, _P, _P, _P, _I64, _P, _P, _I64, _I64, _I, _I, _I,
                                        _I, _I, _I64, _P, _P, _P, _P]),
    "indexer_score_topk_witness": (_I, [_P, _P, _P, _P, _I64, _P, _P, _I64, _I64, _I, _I, _I,
                                        _I, _I, _I64, _P, _I64, _I, _P, _P, _P, _P, _SZ, _P]),
    "indexer_score_topk_varlen": (_I, [_P, _P, _P, _P, _I64, _P, _P, _I64, _I64, _I, _I, _I, _I,
                                       _I, _P, _P, _P, _P, _I, _I64, _P, _P, _P, _P, _SZ, _P]),
    "indexer_workspace_bytes_varlen": (_I, [_P, _I64, _I64, _I, _I, _I, _I, _I, _I64,
                                            ctypes.POINTER(_SZ)]),
    "indexer_pair_overlap": (_I, [_P, _P, _I64, _I, _P, _P]),
    "indexer_pair_regions": (_I, [_P, _P, _I64, _I, _P, _P, _P, _P, _P]),
    "indexer_overlap_summary": (_I, [_P, _P, _I64, ctypes.POINTER(OverlapStats)]),
    "indexer_screen_certificates": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _I, _P, _I64, _I, _I,
                                         _I64, _P, _P, _P, _P, _P, _P, _P]),
    "indexer_strerror": (ctypes.c_char_p, [_I]),
    "indexer_source_hash": (ctypes.c_char_p, []),
}

_lib = None
_lock = threading.Lock()


def load():
    """Load the HIP library; build it first if it has never been built.
    Raises if it cannot be built or loaded, or if it was built from other
    sources than the ones beside it (a stale build): there is no fallback
    path."""
    global _lib
    with _lock:
        if _lib is None:
            from . import build
            if not os.path.exists(LIB_PATH):
                build.build()
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype, fn.argtypes = res, args
            built, want = lib.indexer_source_hash().decode(), build.source_hash()
            if built != want:
                raise RuntimeError(
                    f"{LIB_PATH} was built from other sources (hash {built}) than those in "
                    f"{build.CSRC} (hash {want}); rebuild it with "
                    f"'python -m dsa_indexer_score_amd.build'")
            _lib = lib
    return _lib


def check(code: int, what: str):
    if code != IDX_OK:
        msg = load().indexer_strerror(code).decode()
        raise RuntimeError(f"{what} failed: {msg} (status {code})")
