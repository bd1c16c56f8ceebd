#!/usr/bin/env python3
"""Benchmark of the selective decode-attention step on one MI355X.

A step is one decode step of one attention layer for a batch of sequences:
    block_score (summary mode) -> topk_select -> sparse_decode_attn
over a KV cache whose block summaries were built beforehand (kv_summary_build
runs once per cache, after prefill, and is timed separately).  Inputs are the
seeded synthetic workload (default: batch 32, 32K context, Llama-3.1-8B-shaped
layer, 1 % of the tokens read exactly plus one proxy per unread block), resident
in HBM before the timed region.  Before every step a 1 GiB buffer is written so
that no input is served from the 256 MB last-level cache (cold cache, like a
different layer's cache between two uses); each step is bracketed by HIP events
on the stream the kernels run on, and the flush is outside the events.

Prints one JSON line (see the keys below).  --gpus above 1 is refused: this
build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline decode shape)")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache flush between steps (warm cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU time budget of the oracle baseline")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--traffic", default=None, help="JSON file with measured HBM bytes per attention launch")
    return ap.parse_args()


def algorithmic_bytes(w, m=0):
    """Bytes the sparse step must move per launch (reads, writes), following the read
    accounting of the OpenAttention explainer ('A worked example...' / limits paragraph):
    exact K/V rows of the kept blocks, proxy rows (mean key + mean value) of the other
    blocks, weighted-token rows, the queries, the selection, and the outputs."""
    e = w.elem_bytes
    d, L, k, nb, G = w.head_dim, w.block_size, w.k, w.n_blocks, w.group
    per_read = k * L * 2 * d * e + (nb - k if w.proxies else 0) * 2 * d * e + m * (2 * d * e + 8) + G * d * e + 4 * k
    per_write = G * (d + 1) * 4
    pairs = w.batch * w.n_kv_heads
    return pairs * per_read, pairs * per_write


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the selective decode path has no "
              "multi-GPU mode in this build.", file=sys.stderr)
        sys.exit(2)

    import torch

    from coreset_softmax_attention_amd import csa
    from coreset_softmax_attention_amd import workloads as W

    if not os.path.exists(csa.library_path()):
        from coreset_softmax_attention_amd import build_lib

        build_lib.build()
    w = W.WORKLOADS[args.workload or W.HEADLINE]
    t0 = time.time()
    data = W.generate(w)
    gen_s = time.time() - t0
    print(f"[bench] generated {w.name} in {gen_s:.1f} s", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, K, V = (csa.to_device(data[x], dev) for x in ("q", "K", "V"))
    tok_idx = csa.to_device(data["tok_idx"], dev) if w.coreset else None
    tok_logw = csa.to_device(data["tok_logw"], dev) if w.coreset else None
    m = w.coreset

    # prefill-time summaries (timed for information)
    Kbar, Vbar = csa.kv_summary_build(K, V, w.block_size)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    csa.kv_summary_build(K, V, w.block_size, Kbar, Vbar)
    ev[1].record()
    torch.cuda.synchronize()
    summary_ms = ev[0].elapsed_time(ev[1])

    shape = csa.make_shape(q, K, w.block_size)
    B, Hq, Hkv, nb = w.batch, w.n_q_heads, w.n_kv_heads, w.n_blocks
    scores = torch.empty((B, Hkv, nb), dtype=torch.float32, device=dev)
    sel = torch.empty((B, Hkv, min(w.k, nb)), dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    mode_entry = csa.CSA_WS_BLOCK_SCORE_SUMMARY if w.score_mode == "summary" else csa.CSA_WS_BLOCK_SCORE_EXACT_MASS
    ws_score = torch.empty(max(1, csa.workspace_size(shape, mode_entry)), dtype=torch.uint8, device=dev)
    ws_attn = torch.empty(max(1, csa.workspace_size(shape, csa.CSA_WS_SPARSE_DECODE_ATTN, w.k, m)),
                          dtype=torch.uint8, device=dev)
    keys = Kbar if w.score_mode == "summary" else K
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def step():
        csa.block_score(q, keys, w.score_mode, w.block_size, n_tokens=w.n_tokens, scores=scores, ws=ws_score)
        csa.topk_select(scores, w.k, sel=sel)
        e_mid.record()
        csa.sparse_decode_attn(q, K, V, Kbar, Vbar, sel, w.block_size, proxies=w.proxies, tok_idx=tok_idx,
                               tok_logw=tok_logw, out=out, lse=lse, ws=ws_attn)

    e_mid = torch.cuda.Event(enable_timing=True)
    for i in range(args.warmup):
        if not args.no_flush:
            flush.fill_(i & 0xFF)
        step()
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        if not args.no_flush:
            flush.fill_((i + 1) & 0xFF)
        starts[i].record()
        e_mid = mids[i]
        step()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    attn_ms = np.array([mm.elapsed_time(e) for mm, e in zip(mids, ends)])
    pre_ms = np.array([s.elapsed_time(mm) for s, mm in zip(starts, mids)])
    t_step = float(step_ms.mean())
    t_attn = float(attn_ms.mean())

    rd, wr = algorithmic_bytes(w, m)
    achieved = (rd + wr) / (t_attn * 1e-3) / 1e9
    traffic = None
    if args.traffic and os.path.exists(args.traffic):
        traffic = json.load(open(args.traffic)).get("bytes_per_launch")

    dense_ms = None
    if not args.no_dense:
        ws_dense = torch.empty(max(1, csa.workspace_size(shape, csa.CSA_WS_DENSE_DECODE_ATTN)), dtype=torch.uint8,
                               device=dev)
        dout = torch.empty_like(out)
        dlse = torch.empty_like(lse)
        ts = []
        for i in range(6):
            flush.fill_(i & 0xFF)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            csa.dense_decode_attn(q, K, V, out=dout, lse=dlse, ws=ws_dense)
            b.record()
            torch.cuda.synchronize()
            if i >= 1:
                ts.append(a.elapsed_time(b))
        dense_ms = float(np.mean(ts))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, data, args.cpu_seconds)

    result = {
        "metric": "selective decode attn: queries/s + achieved HBM GB/s, B=32, 32K ctx, 1% read",
        "value": B / (t_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded generator; no dataset or weights)",
        "config": {
            "workload": w.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": w.head_dim,
            "context": w.n_tokens, "block_size": w.block_size, "k_blocks": w.k,
            "exact_read_fraction": w.k * w.block_size / w.n_tokens, "score": w.score_mode, "proxies": w.proxies,
            "weighted_tokens": m, "cache": "warm" if args.no_flush else "cold (1 GiB written before each step)",
        },
        "achieved_hbm_gb_s": achieved,
        "head_queries_per_s": B * Hq / (t_step * 1e-3),
        "step_breakdown_us": {"block_score+topk": float(pre_ms.mean()) * 1e3, "sparse_decode_attn": t_attn * 1e3},
        "step_p10_p90_us": [float(np.percentile(step_ms, 10)) * 1e3, float(np.percentile(step_ms, 90)) * 1e3],
        "wall_s_timed_region_incl_flush": wall,
        "kv_summary_build_ms": summary_ms,
        "dense_decode_attn_ms": dense_ms,
        "sparse_vs_dense_speedup": (dense_ms / t_attn) if dense_ms else None,
        "roofline": {
            "kernel": "sparse_decode_attn",
            "bound": "hbm",
            "achieved": achieved,
            "peak": 8000.0,
            "unit": "GB/s",
            "frac": achieved / 8000.0,
            "traffic": traffic,
            "algorithmic_bytes": rd + wr,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def cpu_baseline(w, data, budget_s):
    """The fp64 oracle's decode step (block score, top-k, attention) on the host cores, on a
    bounded sample of the same workload: the first few sequences of the batch."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from oracle import oracle as O

    nseq = min(4, w.batch)
    sub = {k: v[:nseq] for k, v in data.items()}
    shp = O.Shape(nseq, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_tokens, w.block_size, w.dtype)
    Kbar, Vbar = O.kv_summary_build(shp, sub["K"], sub["V"])  # cache state, not timed
    md = O.SUMMARY if w.score_mode == "summary" else O.EXACT_MASS
    keys = Kbar if w.score_mode == "summary" else sub["K"]
    reps, t0 = 0, time.perf_counter()
    while True:
        score = O.block_score(shp, md, sub["q"], keys)
        sel, _ = O.topk_select(score, w.k)
        O.sparse_decode_attn(shp, sub["q"], sub["K"], sub["V"], Kbar, Vbar, sel, w.proxies,
                             sub.get("tok_idx"), sub.get("tok_logw"))
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 10000:
            break
    cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": nseq * reps / el, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} repetitions of the decode step for the first {nseq} of {w.batch} sequences "
                      f"({el:.1f} s, fp64, OpenMP over KV heads)", "cpu": model}


if __name__ == "__main__":
    main()
