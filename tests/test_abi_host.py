"""C-ABI checks that need no GPU: the library loads, exports every function
include/dsa_indexer.h declares, and its host-side arithmetic and argument
validation behave as documented (nothing here reaches a device call)."""
import ctypes
import os
import re

import numpy as np
import pytest

from dsa_indexer_score_amd import _lib
from oracle import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa_indexer.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*\**\s*(indexer_\w+)\s*\(", text, re.M)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.load()._name)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_output_width_matches_oracle_arithmetic():
    lib = _lib.load()
    W = ctypes.c_int()
    for topk in (1, 4, 64, 512, 2048, 4096):
        for m in (1, 2, 4, 8):
            for flags in (0, _lib.IDX_EXPAND, _lib.IDX_EXPAND | _lib.IDX_TAIL):
                rc = lib.indexer_output_width(topk, m, flags, ctypes.byref(W))
                if (flags & _lib.IDX_EXPAND) and topk % m:
                    assert rc == _lib.IDX_EINVAL
                    continue
                assert rc == 0
                assert W.value == orc.output_width(topk, m, bool(flags & 1), bool(flags & 2))
    assert lib.indexer_output_width(2048, 4, 3, ctypes.byref(W)) == 0 and W.value == 2051
    assert lib.indexer_output_width(8, 4, _lib.IDX_TAIL, ctypes.byref(W)) == _lib.IDX_EINVAL
    assert lib.indexer_output_width(0, 4, 0, ctypes.byref(W)) == _lib.IDX_EINVAL


def _handle(dtype=_lib.IDX_BF16, flags=0, chunk=0, few=0):
    lib = _lib.load()
    h = ctypes.c_void_p()
    cfg = _lib.IndexerConfig(dtype, flags, chunk, few)
    assert lib.indexer_create(ctypes.byref(cfg), 0, ctypes.byref(h)) == 0
    return lib, h


def test_create_rejects_bad_configs():
    lib = _lib.load()
    h = ctypes.c_void_p()
    for dtype, flags, chunk, dev in ((7, 0, 0, 0), (1, 16, 0, 0), (1, _lib.IDX_TAIL, 0, 0),
                                     (1, 0, -1, 0), (1, 0, 0, -1)):
        cfg = _lib.IndexerConfig(dtype, flags, chunk)
        assert lib.indexer_create(ctypes.byref(cfg), dev, ctypes.byref(h)) == _lib.IDX_EINVAL
    assert lib.indexer_create(None, 0, ctypes.byref(h)) == _lib.IDX_EINVAL
    assert lib.indexer_destroy(None) == 0


def test_workspace_bytes_scale_with_chunk_and_selection():
    """Streaming path: candidate buffers for one query chunk."""
    lib, h = _handle(chunk=16384, few=-1)
    n = ctypes.c_size_t()
    assert lib.indexer_workspace_bytes(h, 262144, 65536, 64, 128, 4, 2048, ctypes.byref(n)) == 0
    assert n.value == 16384 * 20736 * 8         # 10 x 2048 + 256 candidate slots of 8 bytes
    assert lib.indexer_workspace_bytes(h, 100, 65536, 64, 128, 4, 2048, ctypes.byref(n)) == 0
    assert n.value == 100 * 20736 * 8           # chunk clipped to S
    assert lib.indexer_workspace_bytes(h, 100, 100, 64, 128, 4, 2048, ctypes.byref(n)) == 0
    assert n.value == 100 * 192 * 8             # never more than all keys plus one tile
    assert lib.indexer_workspace_bytes(h, 100, 10 ** 6, 64, 128, 1, 20000,
                                       ctypes.byref(n)) == _lib.IDX_EUNSUPPORTED
    lib.indexer_destroy(h)


def test_workspace_bytes_automatic_query_chunk():
    """query_chunk = 0 on the streaming path: as many rows as 4 GiB of
    candidate buffers hold at the capacity T allows (a multiple of 8, at
    least 2,048), never more than S."""
    lib, h = _handle(few=-1)
    n = ctypes.c_size_t()
    cap = 10 * 2048 + 256                                  # 20,736 slots of 8 bytes
    rows = (2 ** 32 // (cap * 8)) // 8 * 8                 # 25,888
    assert lib.indexer_workspace_bytes(h, 2 ** 20, 262144, 64, 128, 4, 2048,
                                       ctypes.byref(n)) == 0
    assert n.value == rows * cap * 8 <= 2 ** 32
    assert lib.indexer_workspace_bytes(h, 5000, 262144, 64, 128, 4, 2048, ctypes.byref(n)) == 0
    assert n.value == 5000 * cap * 8
    lib.indexer_destroy(h)


def _capacity(ksel, P):
    """Streaming candidate slots per row (the documented formula)."""
    up = lambda x, a: -(-x // a) * a
    return min(min(up(10 * ksel + 256, 64), 65472), up(max(P, 0), 64) + 64)


def _dense_bytes(S, T, ksel=2048):
    """The documented few-query layout for S rows of at most T keys: key
    sample and witness scores (16384 fp32 per row), estimates, the counts of 32 candidate
    sub-lists, repair marks, the batch directory (8 bytes per 256 keys) and
    the candidate sub-lists (max(32 x 1024, streaming capacity) entries of 8
    bytes), each part 256-byte aligned.  Nothing in it holds a score per
    key."""
    up = lambda x, a: -(-x // a) * a
    nb = -(-max(T, 1) // 256)
    cap = max(32 * 1024, _capacity(ksel, T))
    return up(S * 16384 * 4, 256) + up(S * 4, 256) + up(S * 32 * 4, 256) + up(S * 4, 256) + \
        up(S * nb * 8, 256) + S * cap * 8


def test_workspace_bytes_of_the_few_query_path():
    """At or below few_query_rows (default 1024) the workspace holds the
    rows' key samples, candidate sub-lists and batch directory -- a fixed
    part per row plus 1/32 byte per (row, key), where a score array would be
    4 bytes -- for as many rows as fit in 4 GiB (the rest are taken in
    further passes); a negative setting always streams."""
    n = ctypes.c_size_t()
    lib, h = _handle(chunk=16384)
    assert lib.indexer_workspace_bytes(h, 64, 262144, 64, 128, 4, 2048, ctypes.byref(n)) == 0
    assert n.value == _dense_bytes(64, 262144)
    n4 = ctypes.c_size_t()
    assert lib.indexer_workspace_bytes(h, 64, 4 * 262144, 64, 128, 4, 2048,
                                       ctypes.byref(n4)) == 0
    assert n4.value - n.value == 64 * 3 * 262144 // 256 * 8   # only the directory grows
    assert lib.indexer_workspace_bytes(h, 1, 1001, 64, 128, 4, 2048, ctypes.byref(n)) == 0
    assert n.value == _dense_bytes(1, 1001) == 65536 + 4 * 256 + 32768 * 8
    assert lib.indexer_workspace_bytes(h, 1025, 262144, 64, 128, 4, 2048, ctypes.byref(n)) == 0
    assert n.value == 1025 * 20736 * 8          # above the default: streaming buffers
    assert lib.indexer_workspace_bytes(h, 1024, 262144, 64, 128, 4, 2048, ctypes.byref(n)) == 0
    assert n.value == _dense_bytes(1024, 262144)   # 0.2 GB: one pass
    # 2^31 - 1 keys: the directory alone is 64 MB per row, so 4 GiB holds 63
    # rows and the 64 rows are taken in two passes of 32
    assert lib.indexer_workspace_bytes(h, 64, 2 ** 31 - 1, 64, 128, 1, 2048,
                                       ctypes.byref(n)) == 0
    assert n.value == _dense_bytes(63, 2 ** 31 - 1)
    lib.indexer_destroy(h)
    lib, h = _handle(few=-1)
    assert lib.indexer_workspace_bytes(h, 1, 262144, 64, 128, 4, 2048, ctypes.byref(n)) == 0
    assert n.value == 1 * 20736 * 8
    lib.indexer_destroy(h)
    lib, h = _handle(few=1000)
    assert lib.indexer_workspace_bytes(h, 1000, 4096, 64, 128, 4, 2048, ctypes.byref(n)) == 0
    assert n.value == _dense_bytes(1000, 4096)
    lib.indexer_destroy(h)


def test_few_query_passes_property():
    """For any S and T the few-query workspace holds R rows: the most that
    fit in 4 GiB (at least one, at most S); past one row's fit the call
    streams instead."""
    import random
    rng = random.Random(3)
    lib, h = _handle(few=60000)
    n = ctypes.c_size_t()
    for _ in range(300):
        S, T = rng.randint(1, 3000), rng.choice([rng.randint(1, 5000), rng.randint(1, 1 << 28)])
        assert lib.indexer_workspace_bytes(h, S, T, 8, 64, 1, 64, ctypes.byref(n)) == 0
        lo, hi = 1, S
        while lo < hi:                                         # largest r with r rows fitting
            mid = (lo + hi + 1) // 2
            lo, hi = (mid, hi) if _dense_bytes(mid, T, 64) <= 1 << 32 else (lo, mid - 1)
        R = lo
        assert n.value == _dense_bytes(R, T, 64) <= 1 << 32, (S, T)
    lib.indexer_destroy(h)


def test_workspace_bytes_varlen_follow_the_path():
    """Packed documents: at or below few_query_rows the few-query layout,
    with rows of max_doc_keys scores (0 or above T: T), above it (or with a
    negative setting) the streaming buffers.  The default is 1024 rows with
    at most two rows per document (batched decode), else 64."""
    n = ctypes.c_size_t()
    wb = lambda h, S, T, ndoc, mk: lib.indexer_workspace_bytes_varlen(h, S, T, 64, 128, 4, 2048,
                                                                      ndoc, mk, ctypes.byref(n))
    lib, h = _handle()
    for mk in (0, 4096, 10 ** 9):
        assert wb(h, 8, 4096, 8, mk) == 0
        assert n.value == _dense_bytes(8, 4096)
    assert wb(h, 8, 4096, 8, 1000) == 0
    assert n.value == _dense_bytes(8, 1000)
    assert wb(h, 8, 4096, 8, -1) == _lib.IDX_EINVAL
    assert wb(h, 8, 4096, -1, 0) == _lib.IDX_EINVAL
    assert wb(h, 1025, 4096, 1025, 1000) == 0
    assert n.value == 1025 * (4096 + 64) * 8   # streaming: sized by T
    assert wb(h, 1024, 4096, 512, 1000) == 0   # two rows per document: few-query
    assert n.value == _dense_bytes(1024, 1000)
    assert wb(h, 1024, 4096, 511, 1000) == 0   # more: streaming above 64 rows
    assert n.value == 1024 * (4096 + 64) * 8
    assert wb(h, 64, 4096, 1, 1000) == 0       # at most 64 rows: few-query
    assert n.value == _dense_bytes(64, 1000)
    # 64 decode rows over 64 documents of 262,144 keys: the bound sizes each
    # row's directory (and streaming capacity) by 262,144 keys instead of
    # all 2^24; either way the 64 rows fit in one pass
    T = 64 * 262144
    assert wb(h, 64, T, 64, 262144) == 0
    assert n.value == _dense_bytes(64, 262144)
    assert wb(h, 64, T, 64, 0) == 0
    assert n.value == _dense_bytes(64, T) > _dense_bytes(64, 262144)
    lib.indexer_destroy(h)
    lib, h = _handle(few=-1)
    assert wb(h, 8, 4096, 8, 0) == 0
    assert n.value == 8 * (4096 + 64) * 8
    lib.indexer_destroy(h)


def test_workspace_bytes_with_screening():
    """IDX_SCREEN adds, on the streaming path with 33 <= H <= 64, the
    call's statistics (256 bytes, first), the certificates of one launch's
    rows (1156 bytes a row in five 256-byte aligned parts) and 4 bytes per
    key; H <= 32 cannot screen."""
    up = lambda x, a: -(-x // a) * a
    n = ctypes.c_size_t()
    lib, h = _handle(flags=_lib.IDX_EXPAND | _lib.IDX_TAIL | _lib.IDX_SCREEN, few=-1)
    S, T, cap = 100, 5000, up(5000, 64) + 64          # cap: every visible key fits
    base = S * cap * 8
    want = (up(256 + base, 256) + 2 * up(S * 256, 256) + up(S * 128, 256) + up(S * 4, 256)
            + up(S * 512, 256) + T * 4)
    assert lib.indexer_workspace_bytes(h, S, T, 64, 128, 4, 2048, ctypes.byref(n)) == 0
    assert n.value == want
    assert lib.indexer_workspace_bytes(h, S, T, 32, 128, 4, 2048, ctypes.byref(n)) == 0
    assert n.value == base
    lib.indexer_destroy(h)


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation fails first


def test_screen_certificates_validation():
    """indexer_screen_certificates rejects what it cannot build before any
    device call: H outside 33..64 or an unsupported d, missing pointers, a
    scale that does not match the dtype, misaligned q or k, keys without a
    pointer, a bad visibility rule."""
    lib, h = _handle()
    E, U = _lib.IDX_EINVAL, _lib.IDX_EUNSUPPORTED
    f = lambda **kw: lib.indexer_screen_certificates(
        h, kw.get("q", FAKE), kw.get("qs", None), kw.get("w", FAKE), kw.get("ws", 0),
        kw.get("S", 4), kw.get("H", 64), kw.get("d", 128), kw.get("k", FAKE),
        kw.get("T", 16), kw.get("m", 4), kw.get("causal", 1), kw.get("pos0", 0),
        kw.get("perm", FAKE), kw.get("wv", FAKE), kw.get("wt", FAKE), kw.get("e", FAKE),
        kw.get("agg", FAKE), kw.get("act", None), None)
    assert f(S=0) == 0
    assert f(H=32) == U and f(H=65) == U and f(d=96) == U
    assert f(q=None) == E and f(perm=None) == E and f(e=None) == E and f(agg=None) == E
    assert f(qs=FAKE) == E                                # scales only for fp8
    assert f(q=ctypes.c_void_p(0x10008)) == E
    assert f(k=ctypes.c_void_p(0x10008)) == E
    assert f(k=None) == E                                 # T > 0 keys need a pointer
    assert f(m=0) == E and f(causal=2) == E and f(pos0=-1) == E and f(T=-1) == E
    assert f(ws=10) == E                                  # w rows would overlap
    lib.indexer_destroy(h)
    lib, h = _handle(dtype=_lib.IDX_FP8_E4M3)
    f8 = lambda **kw: lib.indexer_screen_certificates(h, FAKE, kw.get("qs", None), FAKE, 0, 4, 64,
                                                      128, None, 0, 1, 1, 0, FAKE, FAKE, FAKE,
                                                      FAKE, FAKE, None, None)
    assert f8() == E                                      # fp8 needs q_scale
    lib.indexer_destroy(h)


def _call(lib, h, **kw):
    a = dict(q=FAKE, q_scale=None, w=FAKE, w_stride=0, k=FAKE, k_scale=None, S=16, T=16, H=64,
             d=128, m=1, topk=4, causal=1, q_pos0=0, idx=FAKE, vl=FAKE, sel=None, ws=FAKE,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.indexer_score_topk(h, a["q"], a["q_scale"], a["w"], a["w_stride"], a["k"],
                                  a["k_scale"], a["S"], a["T"], a["H"], a["d"], a["m"], a["topk"],
                                  a["causal"], a["q_pos0"], a["idx"], a["vl"], a["sel"], a["ws"],
                                  a["ws_bytes"], a["stream"])


def test_score_topk_validation_paths():
    lib, h = _handle()
    E, U, WS = _lib.IDX_EINVAL, _lib.IDX_EUNSUPPORTED, _lib.IDX_EWORKSPACE
    assert _call(lib, h, S=0) == 0                        # empty problem: nothing to do
    assert _call(lib, h, topk=0) == E
    assert _call(lib, h, m=0) == E
    assert _call(lib, h, causal=2) == E
    assert _call(lib, h, S=-1) == E
    assert _call(lib, h, q_pos0=-1) == E
    assert _call(lib, h, w_stride=3) == E                 # rows of w would overlap
    assert _call(lib, h, q=None) == E
    assert _call(lib, h, idx=None) == E
    assert _call(lib, h, q_scale=FAKE) == E              # scales only for fp8
    assert _call(lib, h, q=ctypes.c_void_p(0x10008)) == E  # misaligned q
    assert _call(lib, h, H=65) == U
    assert _call(lib, h, d=96) == U
    assert _call(lib, h, topk=16001) == U
    assert _call(lib, h, ws=None) == WS
    assert _call(lib, h, ws_bytes=64) == WS
    assert _call(lib, None) == E
    lib.indexer_destroy(h)
    lib, h = _handle(dtype=_lib.IDX_FP8_E4M3)
    assert _call(lib, h) == E                             # fp8 needs scales
    assert _call(lib, h, q_scale=FAKE, k_scale=FAKE, d=96) == U
    lib.indexer_destroy(h)
    lib, h = _handle(flags=_lib.IDX_EXPAND | _lib.IDX_TAIL)
    assert _call(lib, h, m=4, topk=6) == E               # topk not a multiple of m
    assert _call(lib, h, m=4, topk=8, causal=0) == E      # tail needs causal
    assert _call(lib, h, m=4, topk=8, S=64, T=15) == E    # tail needs every complete pool
    lib.indexer_destroy(h)


def test_score_topk_witness_validation_paths():
    """indexer_score_topk_witness validates like indexer_score_topk, plus its
    witness arguments: a negative count, rows that would overlap (stride
    below the count), a missing or misaligned pointer.  No witnesses (count
    0) is a plain call."""
    lib, h = _handle()
    E = _lib.IDX_EINVAL

    def f(wit=FAKE, stride=8, n=8, **kw):
        a = dict(q=FAKE, q_scale=None, w=FAKE, w_stride=0, k=FAKE, k_scale=None, S=16, T=16,
                 H=64, d=128, m=1, topk=4, causal=1, q_pos0=0, idx=FAKE, vl=FAKE, sel=None,
                 ws=FAKE, ws_bytes=1 << 40, stream=None)
        a.update(kw)
        return lib.indexer_score_topk_witness(
            h, a["q"], a["q_scale"], a["w"], a["w_stride"], a["k"], a["k_scale"], a["S"],
            a["T"], a["H"], a["d"], a["m"], a["topk"], a["causal"], a["q_pos0"], wit, stride, n,
            a["idx"], a["vl"], a["sel"], a["ws"], a["ws_bytes"], a["stream"])
    assert f(S=0) == 0
    assert f(n=-1) == E and f(stride=7) == E and f(wit=None) == E
    assert f(wit=ctypes.c_void_p(0x10002)) == E
    assert f(q=None) == E and f(S=-1) == E                 # the plain call's checks remain
    assert f(wit=None, stride=0, n=0, S=0) == 0
    lib.indexer_destroy(h)


def _call_varlen(lib, h, **kw):
    a = dict(q=FAKE, q_scale=None, w=FAKE, w_stride=0, k=FAKE, k_scale=None, S=16, T=16, H=64,
             d=128, m=1, topk=4, causal=1, cu_q=FAKE, cu_k=FAKE, pos0=None, cu_tok=None, ndoc=2,
             max_doc_keys=0, idx=FAKE, vl=FAKE, sel=None, ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.indexer_score_topk_varlen(
        h, a["q"], a["q_scale"], a["w"], a["w_stride"], a["k"], a["k_scale"], a["S"], a["T"],
        a["H"], a["d"], a["m"], a["topk"], a["causal"], a["cu_q"], a["cu_k"], a["pos0"],
        a["cu_tok"], a["ndoc"], a["max_doc_keys"], a["idx"], a["vl"], a["sel"], a["ws"],
        a["ws_bytes"], a["stream"])


def test_score_topk_varlen_validation_paths():
    """Every case is rejected on the host, before any launch."""
    lib, h = _handle()
    E, WS = _lib.IDX_EINVAL, _lib.IDX_EWORKSPACE
    assert _call_varlen(lib, h, S=0) == 0                 # empty problem: nothing to do
    assert _call_varlen(lib, h, max_doc_keys=-1) == E
    assert _call_varlen(lib, h, ndoc=-1) == E
    assert _call_varlen(lib, h, cu_q=None) == E
    assert _call_varlen(lib, h, cu_k=None) == E
    assert _call_varlen(lib, h, ws_bytes=64) == WS
    assert _call_varlen(lib, None) == E
    lib.indexer_destroy(h)
    lib, h = _handle(flags=_lib.IDX_EXPAND | _lib.IDX_TAIL)
    assert _call_varlen(lib, h, m=4, topk=8) == E         # expansion needs cu_tok
    assert _call_varlen(lib, h, m=4, topk=8, cu_tok=FAKE, causal=0) == E  # tail needs causal
    lib.indexer_destroy(h)


def test_pair_overlap_host_paths():
    lib = _lib.load()
    assert lib.indexer_pair_overlap(None, None, 1, 4, None, None) == 0   # no pair
    assert lib.indexer_pair_overlap(None, None, 4, 4, None, None) == _lib.IDX_EINVAL
    assert lib.indexer_pair_overlap(FAKE, FAKE, 4, 0, FAKE, None) == _lib.IDX_EINVAL


def test_overlap_summary_matches_oracle_statistics():
    rng = np.random.default_rng(11)
    lib = _lib.load()
    for S in (2, 7, 1000):
        vl = rng.integers(0, 60, S).astype(np.int32)
        npairs = S // 2
        sh = np.array([rng.integers(0, min(vl[2 * i], vl[2 * i + 1]) + 1) for i in range(npairs)],
                      np.int32)
        st = _lib.OverlapStats()
        assert lib.indexer_overlap_summary(sh.ctypes.data_as(ctypes.c_void_p),
                                           vl.ctypes.data_as(ctypes.c_void_p), S,
                                           ctypes.byref(st)) == 0
        want = orc.overlap_stats(sh, vl)
        assert st.pairs == want["pairs"] and st.excluded == want["excluded"]
        if want["pairs"]:
            for key in ("mean_overlap", "median_overlap", "p90_overlap", "mean_jaccard",
                        "mean_shared", "frac_ge_50", "frac_ge_75", "frac_ge_80"):
                assert getattr(st, key) == pytest.approx(want[key], rel=1e-12, abs=1e-12), key


def test_strerror_is_never_null():
    lib = _lib.load()
    for code in (0, -1, -2, -3, -4, -99):
        assert lib.indexer_strerror(code)


def test_library_was_built_from_these_sources():
    """The loader refuses a library whose embedded source hash differs from
    the sources beside it; the library under test matches them."""
    from dsa_indexer_score_amd import build
    lib = _lib.load()
    assert lib.indexer_source_hash().decode() == build.source_hash()


def test_noalloc_refuses_what_its_scratch_cannot_hold():
    """The no-allocation entry sizes its launches to its static scratch; a
    screened problem whose key norms alone pass it is refused with
    IDX_EWORKSPACE before any device call (host arithmetic only), and the
    message names the limit."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only check; uses placeholder device addresses")
    lib = _lib.load()
    cfg = _lib.IndexerConfig(_lib.IDX_BF16, _lib.IDX_SCREEN, 0, 0)
    h = ctypes.c_void_p()
    assert lib.indexer_create(ctypes.byref(cfg), 0, ctypes.byref(h)) == 0
    fake = ctypes.c_void_p(1 << 20)             # aligned, never dereferenced
    T = 70_000_000                              # 4 T bytes of key norms > 256 MiB
    rc = lib.indexer_score_topk_noalloc(h, fake, None, fake, 0, fake, None, 4096, T, 64, 128, 1,
                                        2048, 0, 0, fake, fake, None, None)
    assert rc == _lib.IDX_EWORKSPACE
    assert "256 MiB" in lib.indexer_strerror(rc).decode()
    # invalid arguments are reported as such, not as a workspace problem
    rc = lib.indexer_score_topk_noalloc(h, fake, None, fake, 0, fake, None, 4096, T, 64, 128, 1,
                                        2048, 2, 0, fake, fake, None, None)
    assert rc == _lib.IDX_EINVAL
    lib.indexer_destroy(h)
