"""Benchmark of the lightning-indexer step on one MI355X.

One step = one pass of the whole hot path over the resident synthetic input:
indexer_score_topk (scoring, streaming top-k, canonical rows, all query
chunks) followed by the adjacent-pair overlap diagnostic.  Inputs are
generated on the device before timing; W warm-up steps run untimed, then
exactly K steps are timed between device synchronisations.

Prints ONE JSON line: whole-job (query, key, head) triples per second, with
queries/s, the MFMA roofline of the scoring kernel (HIP events on the stream
the library launches on), HBM traffic from the committed rocprofv3 counter
summary when it matches the current kernel source, and the CPU oracle timed
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer (q,k,head) triples/s + queries/s at S=256K,H=64; % MFMA peak"
# dense MFMA peaks of the instruction the contraction runs on: e4m3 codes
# widened to bf16 run on the bf16 MFMA, with --fp8-mfma on the fp8 MFMA
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
HBM_PEAK_GBS = 8000.0
KERNEL_SRCS = [os.path.join(ROOT, "dsa_indexer_score_amd", "csrc", f) for f in
               ("score_select.hip", "mfma_ops.h", "select_common.h", "kernels.h")]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "score_select_c4_csa_256k_pmc.md")
# the one-row decode step of the 1M-token workload (few-query path)
DECODE_SRCS = [os.path.join(ROOT, "dsa_indexer_score_amd", "csrc", f) for f in
               ("score_rows.hip", "select_few.hip", "score_select.hip", "mfma_ops.h",
                "select_common.h", "block_cut.h", "kernels.h")]
DECODE_PMC_SUMMARY = os.path.join(ROOT, "profiles", "few_query_decode_c5_csa_1m_pmc.md")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def visible_pairs(S, T, m, causal, q_pos0=0):
    """sum_t P_t, P_t = min(T, (q_pos0 + t + 1) // m) (causal) or T."""
    if not causal:
        return S * T
    total = 0
    # closed form per block of positions sharing floor((p+1)/m)
    p0, p1 = q_pos0, q_pos0 + S  # positions [p0, p1)
    cap_pos = T * m - 1          # from this position on, P = T
    def tri(a, b):  # sum_{p=a}^{b-1} floor((p+1)/m), 0 <= a <= b
        def F(n):   # sum_{x=1}^{n} floor(x/m)
            qn, r = divmod(n, m)
            return m * qn * (qn - 1) // 2 + qn * (r + 1)
        return F(b) - F(a)
    lo = min(p1, max(p0, cap_pos))
    total += tri(p0, lo)
    total += (p1 - lo) * T
    return total


def scored_pairs(S, T, m, causal, ksel, q_pos0=0):
    """Visible pairs of the rows that see more than ksel keys.  Without
    selected scores, a block whose rows all see at most ksel keys writes
    them unscored, so those rows' pairs are not counted as work (a slight
    undercount: a block mixing both kinds scores all its rows)."""
    if T <= ksel:
        return 0
    if not causal:
        return S * T
    first = max(q_pos0, (ksel + 1) * m - 1)  # first position with P > ksel
    if first >= q_pos0 + S:
        return 0
    return visible_pairs(q_pos0 + S - first, T, m, causal, first)


def kernel_sha(srcs=None):
    """sha256[:16] of the sources a kernel is compiled from (default: the
    streaming kernel's)."""
    h = hashlib.sha256()
    for f in srcs or KERNEL_SRCS:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(summary=PMC_SUMMARY, srcs=None, key="traffic_bytes_per_launch"):
    """HBM bytes from a committed counter summary, if it was taken on the
    current kernel sources (else None)."""
    if not os.path.exists(summary):
        return None
    text = open(summary).read()
    sha = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    val = re.search(key + r":\s*([0-9.eE+]+)", text)
    if not sha or not val or sha.group(1) != kernel_sha(srcs):
        return None
    return float(val.group(1))


def gemm_context(dev, n=16384, reps=10):
    """The vendor library's dense bf16 GEMM (torch.matmul, hipBLASLt) on this
    GPU, as a measured reference for the bf16 dense peak: n x n x n on
    normally distributed operands (the data the indexer contracts) and on
    zeros. The matrix units draw more power on random operands, so the
    clock, and with it the attainable fraction of the nominal peak, depends
    on the data."""
    import torch
    g = torch.Generator(device=dev).manual_seed(7)
    out = {"op": "torch.matmul bf16 (hipBLASLt)", "shape": f"{n}x{n}x{n}"}
    for name in ("random_normal", "zeros"):
        if name == "zeros":
            a = torch.zeros(n, n, dtype=torch.bfloat16, device=dev)
            b = torch.zeros(n, n, dtype=torch.bfloat16, device=dev)
        else:
            a = torch.randn(n, n, generator=g, device=dev).to(torch.bfloat16)
            b = torch.randn(n, n, generator=g, device=dev).to(torch.bfloat16)
        c = torch.empty(n, n, dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = 2.0 * n ** 3 / ms / 1e9
        out[f"{name}_tflops"] = tf
        out[f"{name}_frac_of_bf16_peak"] = tf / PEAK_TFLOPS["bf16"]
        del a, b, c
    torch.cuda.empty_cache()
    return out


def cpu_baseline(inp, budget_s, seed, docs=None):
    """The oracle on seeded uniform rows of the same workload, for about
    budget_s seconds of host time; a rate, so no extrapolation is needed.
    With docs (packed documents) the oracle runs per document."""
    from oracle import oracle as orc
    rng = np.random.default_rng(seed)
    # every core this process may run on, up to the host's CPU share for one
    # GPU (OMP_NUM_THREADS where the host sets it, else 16)
    cores = len(os.sched_getaffinity(0))
    share = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    threads = max(1, min(cores, share))
    done_rows, done_triples, spent = 0, 0, 0.0
    while spent < budget_s:
        rows = np.sort(rng.integers(0, inp.S, size=4 * threads))
        t0 = time.perf_counter()
        if docs:
            cq = np.asarray(docs["cu_q_host"])
            p0 = docs.get("pos0_host", np.zeros(len(cq) - 1, np.int64))
            orc.select_rows_varlen(inp, cq, docs["cu_k_host"], rows=rows, nthreads=threads,
                                   pos0=p0, cu_tok=docs.get("cu_tok_host"))
            doc = np.searchsorted(cq, rows, side="right") - 1
            vis = [min(docs["nkeys"][i], (int(p0[i]) + int(r) - int(cq[i]) + 1) // inp.m)
                   for r, i in zip(rows, doc)]
        else:
            orc.select_rows(inp, rows, nthreads=threads)
            vis = [min(inp.T, (int(r) + inp.q_pos0 + 1) // inp.m) if inp.causal else inp.T
                   for r in rows]
        spent += time.perf_counter() - t0
        done_rows += rows.size
        done_triples += sum(vis) * inp.H
    return dict(value=done_triples / spent, unit="triples/s", cores=threads, kind="oracle",
                host_cores=cores, threads=threads,
                sample=f"{done_rows} seeded uniform rows of the {inp.name} workload "
                       f"({done_triples} triples, {spent:.1f} s, fp64, {threads} threads on "
                       f"{cores} available cores)")


def host_streamed(args, inp, ix, W, dev):
    """The workload with q (and its scales) and the outputs in pinned host
    memory: each query chunk is uploaded, scored at its absolute position
    (q_pos0) and its index rows downloaded.  Two buffers per device array
    and one copy stream per direction (default priority) let the upload of
    chunk i+1 and the download of chunk i-1 run while chunk i is scored.
    Device memory then holds the keys, two chunks of q and of idx, and one
    chunk's workspace; the peak is reported beside the step time, which
    includes the PCIe transfers (so it is never the headline)."""
    import torch
    S, chunk = inp.S, inp.query_chunk or inp.S
    q_h = torch.empty(inp.q.shape, dtype=inp.q.dtype, pin_memory=True)
    for r0 in range(0, S, 1 << 16):
        q_h[r0:r0 + (1 << 16)].copy_(inp.q[r0:r0 + (1 << 16)])
    qs_h = None if inp.q_scale is None else inp.q_scale.to("cpu").pin_memory()
    idx_h = torch.empty((S, W), dtype=torch.int32, pin_memory=True)
    vl_h = torch.empty((S,), dtype=torch.int32, pin_memory=True)
    w = inp.w if inp.w.dim() == 1 else None
    if w is None:
        raise SystemExit("--host-streamed takes a broadcast w[H]")
    inp.q = inp.q_scale = None
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    H, d = q_h.shape[1], q_h.shape[2]
    q_d = [torch.empty((chunk, H, d), dtype=q_h.dtype, device=dev) for _ in range(2)]
    qs_d = [None if qs_h is None else torch.empty((chunk, H), dtype=torch.float32, device=dev)
            for _ in range(2)]
    idx_d = [torch.empty((chunk, W), dtype=torch.int32, device=dev) for _ in range(2)]
    vl_d = [torch.empty((chunk,), dtype=torch.int32, device=dev) for _ in range(2)]
    ws = torch.empty((ix.workspace_bytes(chunk, inp.T, H, d, inp.m, inp.topk),), dtype=torch.uint8,
                     device=dev)
    comp = torch.cuda.current_stream(dev)
    up, down = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    starts = list(range(0, S, chunk))
    ev = lambda: [torch.cuda.Event() for _ in range(2)]
    up_done, comp_done, down_done = ev(), ev(), ev()

    def upload(i):
        b, r0 = i % 2, starts[i]
        n = min(chunk, S - r0)
        with torch.cuda.stream(up):
            if i >= 2:
                up.wait_event(comp_done[b])          # chunk i-2 no longer reads q_d[b]
            q_d[b][:n].copy_(q_h[r0:r0 + n], non_blocking=True)
            if qs_h is not None:
                qs_d[b][:n].copy_(qs_h[r0:r0 + n], non_blocking=True)
            up_done[b].record(up)

    def step():
        upload(0)
        for i, r0 in enumerate(starts):
            b, n = i % 2, min(chunk, S - r0)
            if i + 1 < len(starts):
                upload(i + 1)
            comp.wait_event(up_done[b])
            if i >= 2:
                comp.wait_event(down_done[b])        # idx_d[b] of chunk i-2 downloaded
            ix.score_topk(q_d[b][:n], w, inp.k, m=inp.m, topk=inp.topk, causal=inp.causal,
                          q_scale=None if qs_h is None else qs_d[b][:n], k_scale=inp.k_scale,
                          q_pos0=r0, workspace=ws, out=(idx_d[b][:n], vl_d[b][:n], None))
            comp_done[b].record(comp)
            with torch.cuda.stream(down):
                down.wait_event(comp_done[b])
                idx_h[r0:r0 + n].copy_(idx_d[b][:n], non_blocking=True)
                vl_h[r0:r0 + n].copy_(vl_d[b][:n], non_blocking=True)
                down_done[b].record(down)
        comp.wait_stream(down)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    peak = torch.cuda.max_memory_allocated(dev)
    print(json.dumps({
        "metric": "host-streamed indexer step: peak device bytes and PCIe-inclusive time",
        "workload": inp.name, "S": S, "T": inp.T, "query_chunk": chunk, "steps": args.steps,
        "ms_per_step": ms, "peak_hbm_bytes_allocated": int(peak),
        "queries_per_s": S / (ms / 1e3),
        "transfers_per_step_bytes": int(q_h.numel() * q_h.element_size() +
                                        (0 if qs_h is None else qs_h.numel() * 4) +
                                        idx_h.numel() * 4 + vl_h.numel() * 4)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="c4_csa_256k")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm-context", action="store_true",
                    help="skip timing the vendor bf16 GEMM beside the prefill kernel")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain device copy of known size (counter calibration)")
    ap.add_argument("--varlen", type=int, default=0, metavar="N",
                    help="pack the workload's sequence as N equal documents (per-document "
                         "pools, causality and keys) and time the varlen entry point")
    ap.add_argument("--regions", action="store_true",
                    help="also time the three-region q-cluster split of the adjacent pairs")
    ap.add_argument("--wdist", default=None, choices=["normal_bcast", "lognormal_bcast"],
                    help="override the workload's head-weight distribution")
    ap.add_argument("--graph", action="store_true",
                    help="capture the step in HIP graphs once and time replays")
    ap.add_argument("--screen", action="store_true",
                    help="DoSA certificate screening on the streaming path (lossless)")
    ap.add_argument("--decode-batch", type=int, default=0, metavar="B",
                    help="batched decode: B documents of the workload's full context packed "
                         "together, one query row at the end of each (varlen entry point)")
    ap.add_argument("--few-query-rows", type=int, default=None,
                    help="override indexer_config.few_query_rows (negative: never)")
    ap.add_argument("--S", type=int, default=0, metavar="ROWS",
                    help="prefill sweep: the workload scaled to ROWS queries (keys follow)")
    ap.add_argument("--topk", type=int, default=0, help="override the workload's top-k")
    ap.add_argument("--chunk", type=int, default=0, help="override the query chunk")
    ap.add_argument("--context", type=int, default=0, metavar="TOKENS",
                    help="--decode: a context of TOKENS tokens instead of the workload's")
    ap.add_argument("--host-streamed", action="store_true",
                    help="q in pinned host memory, uploaded per query chunk; idx chunks "
                         "downloaded: reports peak device bytes and the PCIe-inclusive time")
    ap.add_argument("--fp8-mfma", action="store_true",
                    help="e4m3 workloads: contract the codes on the fp8 MFMA (IDX_FP8_MFMA)")
    ap.add_argument("--heads", type=int, default=0, metavar="H",
                    help="override the workload's head count (1..64)")
    ap.add_argument("--witness", action="store_true",
                    help="--decode: each row's witnesses are the selection of the row one "
                         "position earlier (the previous decode step)")
    ap.add_argument("--rho", type=float, default=None,
                    help="AR(1) correlation of adjacent queries (default: the workload's)")
    ap.add_argument("--decode", type=int, default=0, metavar="N",
                    help="few-query shape: N query rows at the end of the workload's full "
                         "context (every key visible), timed through the few-query path")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(see the sharding note in the design document).", file=sys.stderr)
        sys.exit(2)

    import torch

    import dsa_indexer_score_amd as dsai
    from workloads import gen

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"bench: library {dsai.library_path()}")
    t0 = time.perf_counter()
    over = {"wdist": args.wdist} if args.wdist else {}
    if args.heads:
        over["H"] = args.heads
    if args.decode_batch:
        from dataclasses import replace
        full_T = gen.CONFIGS[args.workload]["T"]
        inp = gen.generate(args.workload, S=args.decode_batch, T=args.decode_batch * full_T,
                           device=dev, **over)
        inp = replace(inp, query_chunk=None)
    elif args.decode:
        from dataclasses import replace
        m = gen.CONFIGS[args.workload]["m"]
        full_T = args.context // m if args.context else gen.CONFIGS[args.workload]["T"]
        if args.rho is not None:
            over["rho"] = args.rho
        # --witness: one more row first; it is selected untimed and its
        # selection is the next row's witnesses (the previous decode step)
        S_gen = args.decode + (1 if args.witness else 0)
        inp = gen.generate(args.workload, S=S_gen, T=full_T, device=dev, **over)
        inp = replace(inp, q_pos0=full_T * inp.m - S_gen, query_chunk=None)
    else:
        inp = gen.generate(args.workload, S=args.S or None, topk=args.topk or None,
                           device=dev, **over)
    if args.chunk:
        from dataclasses import replace
        inp = replace(inp, query_chunk=args.chunk)
    torch.cuda.synchronize()
    log(f"bench: generated {args.workload} S={inp.S} T={inp.T} H={inp.H} d={inp.d} m={inp.m} "
        f"topk={inp.topk} dtype={inp.dtype} chunk={inp.query_chunk} in "
        f"{time.perf_counter() - t0:.1f} s")

    few = max(64, args.decode, args.decode_batch) if (args.decode or args.decode_batch) else 0
    if args.few_query_rows is not None:
        few = args.few_query_rows
    ix = dsai.Indexer(inp.q.dtype, expand=inp.expand, tail=inp.tail,
                      query_chunk=inp.query_chunk or 0, few_query_rows=few,
                      screen=args.screen, fp8_mfma=args.fp8_mfma, device=dev)
    W = dsai.output_width(inp.topk, inp.m, inp.expand, inp.tail)
    ksel = inp.topk // inp.m if inp.expand else inp.topk
    witness = None
    if args.witness:
        if not args.decode:
            raise SystemExit("--witness applies to --decode")
        from dataclasses import replace
        prev_w = inp.w if inp.w.dim() == 1 else inp.w[:-1]
        witness = ix.score_topk(inp.q[:-1], prev_w, inp.k, m=inp.m, topk=inp.topk,
                                causal=inp.causal,
                                q_scale=None if inp.q_scale is None else inp.q_scale[:-1],
                                k_scale=inp.k_scale, q_pos0=inp.q_pos0)[0]
        inp = replace(inp, q=inp.q[1:].contiguous(), S=inp.S - 1, q_pos0=inp.q_pos0 + 1,
                      q_scale=None if inp.q_scale is None else inp.q_scale[1:].contiguous(),
                      w=inp.w if inp.w.dim() == 1 else inp.w[1:].contiguous())
        torch.cuda.synchronize()
    docs = None
    if args.varlen:
        # N equal documents; document i owns rows [i*L, (i+1)*L) and its own
        # L // m complete pools (the last document takes the remainder)
        L = inp.S // args.varlen
        lens = [L] * (args.varlen - 1) + [inp.S - L * (args.varlen - 1)]
        nkeys = [n // inp.m for n in lens]
        cu_q = np.concatenate([[0], np.cumsum(lens)])
        cu_k = np.concatenate([[0], np.cumsum(nkeys)])
        if cu_k[-1] > inp.T:
            raise SystemExit("the workload has fewer keys than its documents' pools")
        t32 = lambda a: torch.as_tensor(np.asarray(a), dtype=torch.int32, device=dev)
        docs = dict(cu_q=t32(cu_q), cu_k=t32(cu_k), cu_tok=t32(cu_q[:-1]) if inp.expand else None,
                    lens=lens, nkeys=nkeys, cu_q_host=cu_q, cu_k_host=cu_k,
                    cu_tok_host=cu_q[:-1] if inp.expand else None,
                    pairs=sum(scored_pairs(n, k, inp.m, inp.causal, ksel)
                              for n, k in zip(lens, nkeys)))
    if args.decode_batch:
        # document i: keys [i*T_doc, (i+1)*T_doc), one row at its last token
        B, T_doc = args.decode_batch, inp.T // args.decode_batch
        cu_q = np.arange(B + 1)
        cu_k = np.arange(B + 1) * T_doc
        pos0 = np.full(B, T_doc * inp.m - 1, np.int64)
        cu_tok = np.arange(B) * T_doc * inp.m
        t32 = lambda a: torch.as_tensor(np.asarray(a), dtype=torch.int32, device=dev)
        docs = dict(cu_q=t32(cu_q), cu_k=t32(cu_k), cu_tok=t32(cu_tok) if inp.expand else None,
                    pos0=torch.as_tensor(pos0, device=dev), lens=[1] * B, nkeys=[T_doc] * B,
                    cu_q_host=cu_q, cu_k_host=cu_k, pos0_host=pos0,
                    cu_tok_host=cu_tok if inp.expand else None,
                    pairs=B * (min(T_doc, T_doc * inp.m // inp.m) if inp.causal else T_doc))
    if args.host_streamed:
        host_streamed(args, inp, ix, W, dev)
        return
    idx = torch.empty((inp.S, W), dtype=torch.int32, device=dev)
    vl = torch.empty((inp.S,), dtype=torch.int32, device=dev)
    # packed documents: the longest document's keys bound the dense rows
    max_doc_keys = int(max(docs["nkeys"])) if docs else 0
    nbytes = (ix.workspace_bytes_varlen(inp.S, inp.T, inp.H, inp.d, inp.m, inp.topk,
                                        len(docs["nkeys"]), max_doc_keys) if docs else
              ix.workspace_bytes(inp.S, inp.T, inp.H, inp.d, inp.m, inp.topk))
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def score():
        if docs:
            ix.score_topk_varlen(inp.q, inp.w, inp.k, docs["cu_q"], docs["cu_k"], m=inp.m,
                                 topk=inp.topk, causal=inp.causal, pos0=docs.get("pos0"),
                                 cu_tok=docs["cu_tok"], q_scale=inp.q_scale,
                                 k_scale=inp.k_scale, max_doc_keys=max_doc_keys,
                                 workspace=ws, out=(idx, vl, None))
        else:
            ix.score_topk(inp.q, inp.w, inp.k, m=inp.m, topk=inp.topk, causal=inp.causal,
                          q_scale=inp.q_scale, k_scale=inp.k_scale, q_pos0=inp.q_pos0,
                          workspace=ws, out=(idx, vl, None), witness=witness)

    if args.graph:
        # The step captured once (score_topk and pair_overlap as two graphs,
        # so each can be timed) and replayed: no host work per step.
        score()
        torch.cuda.synchronize()
        g_score, g_ovl = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_score):
            score()
        with torch.cuda.graph(g_ovl):
            shared_g = dsai.pair_overlap(idx, vl)
        score, overlap = g_score.replay, lambda: (g_ovl.replay(), shared_g)[1]
    else:
        def overlap():
            return dsai.pair_overlap(idx, vl)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        score()
        if ev:
            ev[1].record(stream)
        shared = overlap()
        if ev:
            ev[2].record(stream)
        return shared

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        shared = step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    score_ms = [e[0].elapsed_time(e[1]) for e in evs]
    ovl_ms = [e[1].elapsed_time(e[2]) for e in evs]
    peak_bytes = torch.cuda.max_memory_allocated(dev)

    ms_per_step = wall * 1e3 / args.steps
    if docs:
        pairs = docs["pairs"]
    elif args.decode:
        pairs = visible_pairs(inp.S, inp.T, inp.m, inp.causal, inp.q_pos0)  # dense: all scored
    else:
        pairs = scored_pairs(inp.S, inp.T, inp.m, inp.causal, ksel, inp.q_pos0)
    triples = pairs * inp.H
    flops = 2 * inp.d * triples
    n_launch = math.ceil(inp.S / (inp.query_chunk or inp.S))
    score_s = float(np.mean(score_ms)) / 1e3
    achieved_tflops = flops / score_s / 1e12
    # the instruction the contraction runs on, and its dense peak
    mfma_dtype = {"bf16": "bf16", "f32": "f32",
                  "fp8": "fp8" if args.fp8_mfma and inp.d in (64, 128) and not args.screen
                  else "bf16"}[inp.dtype]
    peak = PEAK_TFLOPS[mfma_dtype]
    # the committed counters are for the default 256K-query workload only
    default_run = (args.workload == "c4_csa_256k" and not (
        args.decode or args.decode_batch or args.varlen or args.screen or args.heads or args.S
        or args.topk or args.chunk or args.wdist or args.fp8_mfma or args.graph))
    traffic = stored_traffic() if default_run else None

    screen_stats = None
    if args.screen and not docs and not args.decode:
        # the last call's counts, at the start of its workspace
        tested, passed = ws[:16].view(torch.int64).cpu().tolist()
        screen_stats = {"keys_tested": tested, "keys_passed": passed,
                        "survival": passed / tested if tested else None}
    st = dsai.overlap_summary(shared, vl)
    regions = None
    if args.regions:
        # fixed-capacity outputs: 2 rows read, 3 rows + 3 counts written per pair
        W_ = idx.shape[1]
        npairs = inp.S // 2
        rb = npairs * (2 * W_ * 4 + 2 * 4 + 3 * W_ * 4 + 3 * 4)
        for _ in range(2):
            dsai.pair_regions(idx, vl)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            dsai.pair_regions(idx, vl)
        e1.record(stream)
        torch.cuda.synchronize()
        rms = e0.elapsed_time(e1) / 10
        regions = {"ms": rms, "bytes": rb, "GB/s": rb / rms / 1e6,
                   "frac_of_hbm": rb / rms / 1e6 / HBM_PEAK_GBS}
    if args.copy_calibration:
        # One elementwise kernel of known size (reads 1 GiB, writes 1 GiB): the
        # scale for the FETCH_SIZE / WRITE_SIZE counters of the same run.
        a = torch.ones(256 << 20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        log("bench: copy calibration: 1 GiB read + 1 GiB written (neg kernel)")

    workload_name = inp.name
    if args.decode:
        workload_name = f"{inp.name} decode: {inp.S} rows at positions " \
                        f"{inp.q_pos0}..{inp.q_pos0 + inp.S - 1}"
    if args.varlen:
        workload_name = f"{inp.name} packed as {args.varlen} documents of {docs['lens'][0]} " \
                        f"tokens (varlen)"
    if args.decode_batch:
        workload_name = f"{inp.name} batched decode: {args.decode_batch} documents of " \
                        f"{inp.T // args.decode_batch} keys, one row at the end of each (varlen)"
    roofline = {"bound": "mfma", "achieved": achieved_tflops, "peak": peak,
                "unit": "TFLOP/s", "frac": achieved_tflops / peak,
                "traffic": None if traffic is None else traffic,
                "kernel": "score_select", "flops_per_launch": flops / n_launch,
                "avg_launch_ms": score_s * 1e3 / n_launch,
                "mfma_dtype": mfma_dtype}
    if inp.dtype == "fp8":
        # the fp8 workloads' target is the fp8 dense peak, whatever MFMA runs
        roofline["frac_of_fp8_peak"] = achieved_tflops / PEAK_TFLOPS["fp8"]
    if args.decode or args.decode_batch:
        # Few-query step (sampled estimate, scoring with sparse write-back,
        # exact cut, repair launch): bound by reading the key set once from
        # HBM.
        esz = {"bf16": 2, "fp8": 1, "f32": 4}[inp.dtype]
        W = dsai.output_width(inp.topk, inp.m, inp.expand, inp.tail)
        alg_bytes = (inp.T * inp.d * esz + inp.S * inp.H * inp.d * esz + inp.w.numel() * 4 +
                     (inp.T * 4 + inp.S * inp.H * 4 if inp.dtype == "fp8" else 0) +
                     inp.S * (W + 1) * 4)
        gbs = alg_bytes / score_s / 1e9
        dtraffic = None
        if (args.workload == "c5_csa_1m" and args.decode == 1 and not args.wdist and
                not args.witness and args.rho is None):
            dtraffic = stored_traffic(DECODE_PMC_SUMMARY, DECODE_SRCS, "traffic_bytes_per_step")
        roofline = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": gbs / HBM_PEAK_GBS, "traffic": dtraffic,
                    "kernel": "few-query step (sample, estimate, filtered scoring, cut, "
                              "repair)",
                    "bytes_per_launch": alg_bytes, "avg_launch_ms": score_s * 1e3,
                    "mfma_frac": achieved_tflops / peak}
    result = {
        "metric": METRIC,
        "value": triples / (ms_per_step / 1e3),
        "unit": "triples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic (seeded, generated on device; no datasets or weights)",
        "config": {"workload": workload_name, "S": inp.S, "T": inp.T, "H": inp.H, "d": inp.d,
                   "m": inp.m, "topk": inp.topk, "causal": inp.causal, "query_chunk":
                   inp.query_chunk, "launches_per_step": n_launch, "screen": bool(args.screen),
                   "wdist": inp.meta.get("wdist"), "graph": bool(args.graph),
                   "fp8_mfma": bool(args.fp8_mfma), "witness": bool(args.witness),
                   "rho": args.rho,
                   "parallelism": "none (1 GPU)"},
        "queries_per_s": inp.S / (ms_per_step / 1e3),
        "mfma_frac": achieved_tflops / peak,
        "score_select_ms": float(np.mean(score_ms)),
        "pair_overlap_ms": float(np.mean(ovl_ms)),
        "peak_hbm_bytes_allocated": int(peak_bytes),
        "roofline": roofline,
        "overlap": {k: st[k] for k in ("mean_overlap", "median_overlap", "mean_jaccard")},
        **({"pair_regions": regions} if regions else {}),
        **({"screen_stats": screen_stats} if screen_stats else {}),
    }
    if not (args.no_gemm_context or args.decode or args.decode_batch or args.host_streamed):
        result["gemm_context"] = gemm_context(dev)
        log(f"bench: vendor bf16 GEMM {result['gemm_context']['random_normal_tflops']:.0f} "
            f"TFLOP/s on normal operands, {result['gemm_context']['zeros_tflops']:.0f} on zeros")
    if not args.no_cpu_baseline:
        log(f"bench: timing the CPU oracle for ~{args.cpu_budget:.0f} s")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget, inp.seed, docs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
