#!/usr/bin/env python3
"""Benchmark of the selective decode-attention step on one MI355X.

A step is one decode step of one attention layer for a batch of sequences:
    block_score (summary mode) -> topk_select -> sparse_decode_attn
over a KV cache whose block summaries were built beforehand (kv_summary_build
runs once per cache after prefill; it is timed separately for information).
The step runs through selective_decode_step, which does the three in one
kernel per KV head for this shape; the same step through the three separate
entry points is timed too ("modular").

Cold cache without flushing: the inputs are replicated into NL independent
caches resident in HBM (like NL layers of a model) and consecutive steps use
consecutive layers, so between two uses of one layer's data the step touches
NL - 1 other layers' data (about 1 GB for the default shape, four times the
256 MB last-level cache).  The default run:
  * eager: K steps, one Python call per entry point, HIP events around the
    whole loop;
  * graph: K decode steps (layers cycled) captured once in a HIP graph and
    replayed (the way a serving loop runs decode); each timed window is one
    replay, i.e. exactly K steps, started behind a GPU sleep so that the host's
    submission is not timed; the median of --windows windows is reported;
  * attention only: the same with K sparse_decode_attn launches, for the
    roofline figure of that kernel on its own.
`value` is queries/s of the graph-replayed step (one query = one sequence's
decode token through the layer, all query heads); the roofline object is for
the step's kernel (bytes: every mean key, the mean values of unread blocks,
the exact key/value rows, the queries and the outputs).

Prints one JSON line.  --gpus above 1 is refused: the selective decode path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline decode shape)")
    ap.add_argument("--layers", type=int, default=8, help="independent cache copies cycled through")
    ap.add_argument("--windows", type=int, default=15,
                    help="timed windows of exactly --steps graph-replayed steps each (the median is reported)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU time budget of the oracle baseline")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--traffic", default=None,
                    help="JSON file with measured HBM bytes per launch (default: profiles/traffic_<workload>.json)")
    ap.add_argument("--counters", nargs=4, default=None,
                    metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB", "COPY_WRITE_DB"),
                    help="only turn four rocprofv3 --pmc result databases (FETCH_SIZE and WRITE_SIZE of a "
                         "run of this script, then of --copy-probe) into the traffic file given by --traffic")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 8 times (calibrates memory counters)")
    return ap.parse_args()


HERE = os.path.dirname(os.path.abspath(__file__))
COPY_PROBE_BYTES = 1 << 30
# kernels whose HBM traffic is reported, by the name rocprofv3 records
TRAFFIC_KERNELS = {"decode_step": "decode_step_kernel", "sparse_decode_attn": "attn_mfma_kernel",
                   "cluster_decode_attn": "cluster_attn_kernel", "cluster_logits": "cluster_logits_kernel",
                   "block_score_exact": "logits_exact_mfma_kernel", "block_score_exact_valu": "logits_exact_kernel",
                   "score_logits_split": "score_logits_split_kernel", "score_finish": "score_finish_kernel",
                   "attn_merge": "attn_merge_kernel", "topk": "topk_", "score_group_chunk": "score_group_chunk_kernel",
                   "block_score_box": "score_summary_fused_kernel<256, true>",
                   "block_score_cobs2_split": "score_cobs2_split_kernel",
                   "block_score_cobs2_fused": "score_cobs2_fused_kernel",
                   "block_score_cobs2_sub": "score_cobs2_sub_fused_kernel", "block_score_err": "score_err_fused_kernel"}
# the kernels of the three-call route (block_score, topk_select, sparse_decode_attn) whose
# measured bytes add up to a step's traffic
THREE_CALL_KERNELS = ("block_score_box", "block_score_cobs2_split", "block_score_cobs2_fused", "block_score_cobs2_sub",
                      "block_score_err", "score_finish", "topk", "sparse_decode_attn")


# The device sources each counted kernel is compiled from (its traffic is stale once any of
# them changes; the host-side declarations in launch.hpp and api.hip do not count).
_DEVICE_COMMON = ["device.hpp", "select.hpp", "attn_engine.hpp"]
KERNEL_SOURCES = {"decode_step": ["step.hip"], "sparse_decode_attn": ["attn.hip"],
                  "cluster_decode_attn": ["cluster.hip"], "cluster_logits": ["cluster.hip"],
                  "block_score_exact": ["score.hip"], "block_score_exact_valu": ["score.hip"],
                  "score_logits_split": ["score.hip"], "score_finish": ["score.hip"], "attn_merge": ["attn.hip"],
                  "topk": ["topk.hip"], "score_group_chunk": ["score.hip"], "block_score_box": ["score.hip"],
                  "block_score_cobs2_split": ["score.hip"], "block_score_cobs2_fused": ["score.hip"],
                  "block_score_cobs2_sub": ["score.hip"], "block_score_err": ["score.hip"]}


def source_hash(csrc=None, files=None):
    """Hash of the HIP sources' code (comments and whitespace dropped), of the files named
    (else of all of them): a traffic figure measured on other code is stale."""
    import glob
    import hashlib
    import re

    h = hashlib.sha256()
    csrc = csrc or os.path.join(HERE, "coreset_softmax_attention_amd", "csrc")
    names = sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.hpp")))
    if files is not None:
        names = [os.path.join(csrc, f) for f in sorted(set(files) | set(_DEVICE_COMMON))]
    for f in names:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            code = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def default_traffic_path(workload):
    return os.path.join(HERE, "profiles", f"traffic_{workload}.json")


def counters_to_traffic(fetch_db, write_db, copy_fetch_db, copy_write_db, out_path, workload):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each reported kernel, scaled by
    what the same counters read for a plain copy of COPY_PROBE_BYTES bytes."""
    import sqlite3

    def per_dispatch(db, counter, name_part):
        con = sqlite3.connect(db)
        rows = con.execute("select name, counter_value from pmc_events where counter_name = ?", (counter,)).fetchall()
        con.close()
        vals = [v for n, v in rows if name_part in n]
        if not vals:
            return None, 0
        return sum(vals) / len(vals), len(vals)

    copy_fetch, _ = per_dispatch(copy_fetch_db, "FETCH_SIZE", "copyBuffer")
    copy_write, _ = per_dispatch(copy_write_db, "WRITE_SIZE", "copyBuffer")
    if copy_fetch is None or copy_write is None:
        raise SystemExit("the copy-probe runs hold no copyBuffer dispatch")
    fetch_scale = COPY_PROBE_BYTES / (copy_fetch * 1024.0)
    write_scale = COPY_PROBE_BYTES / (copy_write * 1024.0)
    kernels = {}
    for key, name in TRAFFIC_KERNELS.items():
        f, nf = per_dispatch(fetch_db, "FETCH_SIZE", name)
        w, nw = per_dispatch(write_db, "WRITE_SIZE", name)
        if f is None or w is None:  # not run by this workload
            continue
        kernels[key] = {"kernel": name, "fetch_kib": f, "write_kib": w, "dispatches": [nf, nw],
                        "bytes": f * 1024.0 * fetch_scale + w * 1024.0 * write_scale,
                        "source_hash": source_hash(files=KERNEL_SOURCES[key])}
    rec = {"workload": workload, "source_hash": source_hash(),
           "copy_probe": {"bytes": COPY_PROBE_BYTES, "fetch_kib": copy_fetch, "write_kib": copy_write,
                          "fetch_scale": fetch_scale, "write_scale": write_scale},
           "kernels": kernels,
           "bytes_per_launch": {k: v["bytes"] for k, v in kernels.items()}}
    if not kernels:
        raise SystemExit(f"{fetch_db}: none of the reported kernels ran")
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec["bytes_per_launch"]))


def load_traffic(path):
    """Measured bytes per launch of the kernels whose device sources are unchanged since (the
    others are left out, reported as null), or None when there is no record."""
    if not path or not os.path.exists(path):
        return None
    rec = json.load(open(path))
    out = {}
    for key, k in rec.get("kernels", {}).items():
        if key in KERNEL_SOURCES and k.get("source_hash") == source_hash(files=KERNEL_SOURCES[key]):
            out[key] = k["bytes"]
        else:
            print(f"[bench] {path}: {key} was measured on other kernel sources: traffic not reported",
                  file=sys.stderr)
    return out


def three_call_traffic(traffic):
    """HBM bytes of one step through block_score, topk_select and sparse_decode_attn: the sum
    of the measured bytes per launch of the kernels of that route (null unless the score
    kernel, the top-k and the attention were all measured on the current sources)."""
    if not isinstance(traffic, dict):
        return None
    keys = [k for k in THREE_CALL_KERNELS if k in traffic]
    if "sparse_decode_attn" not in keys or "topk" not in keys or not any(k.startswith("block_score_") for k in keys):
        return None
    return sum(traffic[k] for k in keys)


def copy_probe(nbytes):
    """A plain device-to-device copy of known size, for scaling hardware byte counters."""
    import torch

    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(8):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": 8}), flush=True)


def step_kernels(w):
    """Which kernels selective_decode_step runs for workload w: the library takes one kernel per
    KV head for summary scores in bfloat16 with G <= 8, k <= 32 and nb <= 2048 when there are at
    least 32 KV heads or each one's share is small ((proxies + k L + m) G <= 4096 with nb <= 512),
    else the split kernels.  Used for the label of the roofline entry only."""
    nb, k = w.n_blocks, min(w.k, w.n_blocks)
    rows = (nb - k if w.proxies else 0) + k * w.block_size + w.coreset
    one = (w.score_mode == "summary" and w.dtype == "bf16" and w.group <= 8 and k <= 32 and nb <= 2048
           and (w.batch * w.n_kv_heads >= 32 or (rows * w.group <= 4096 and nb <= 512)))
    if one:
        return "selective_decode_step (decode_step_kernel)"
    if w.score_mode == "summary" and w.dtype == "bf16" and w.group <= 8 and nb > 512 and 1 <= k <= 32:
        return ("selective_decode_step (split logits, chunk group scores and candidates, attention ranking the "
                "candidates, merge)")
    return "selective_decode_step (the block_score, topk_select and sparse_decode_attn kernels in turn)"


def cluster_step_kernels(w):
    """Which kernels cluster_decode_step runs for workload w: one kernel per KV head in bfloat16
    with G <= 8, k <= 32, at least 32 KV heads and the logits, scores, selection bits and ranges
    of C clusters within 64 KiB of LDS, else cluster_score, topk_select and cluster_decode_attn
    in turn.  Used for the roofline label only."""
    C, G, k = w.qgc, w.group, min(w.k, w.qgc)
    ls = (C + 31) // 32 * 32
    lds = (G + 1) * ls * 4 + ls // 32 * 4 + (ls + 1) * 4
    one = w.dtype == "bf16" and G <= 8 and k <= 32 and C <= 2048 and w.batch * w.n_kv_heads >= 32 and lds <= 65536
    return ("cluster_decode_step (decode_step_kernel over clusters)" if one else
            "cluster_decode_step (the cluster_score, topk_select and cluster_decode_attn kernels in turn)")


def algorithmic_bytes(w, m=0):
    """Bytes the sparse attention must move per launch (reads, writes), following the read
    accounting of the OpenAttention explainer (exact rows, proxy rows and query-side data):
    exact K/V rows of the kept blocks, mean key + mean value rows of the other blocks,
    weighted-token rows (+ index and log-weight), the queries, the selection, the outputs."""
    e = w.elem_bytes
    d, L, k, nb, G = w.head_dim, w.block_size, w.k, w.n_blocks, w.group
    per_read = k * L * 2 * d * e + (nb - k if w.proxies else 0) * 2 * d * e + m * (2 * d * e + 8) + G * d * e + 4 * k
    per_write = G * (d + 1) * 4
    pairs = w.batch * w.n_kv_heads
    return pairs * per_read, pairs * per_write


def step_bytes(w, m=0):
    """Bytes one selective decode step must move (reads, writes).  Summary scores: every mean
    key once (it ranks the blocks and gives the proxy logits), the mean values of the unread
    blocks and the exact key/value rows of the kept blocks.  Exact-mass scores: every key
    once, the values of the kept blocks, both mean rows of the unread blocks.  Box scores:
    both box rows of every block, both mean rows of the unread blocks, the exact rows.
    Proxy-error and second-order scores: the descriptor of every block (mean and variance
    rows; mean and four eigenvector rows, bfloat16 or FP4 with scales), whose mean row
    also gives the proxy logits, then the mean values of the unread blocks and the exact
    rows (the three-call route reads the mean keys a second time: not counted).  Plus
    weighted-token rows, the queries, and the outputs with their log-normalisers."""
    e = w.elem_bytes
    d, L, k, nb, G = w.head_dim, w.block_size, w.k, w.n_blocks, w.group
    unread = (nb - k) if w.proxies else 0
    if w.score_mode == "summary":
        per_read = nb * d * e + unread * d * e + k * L * 2 * d * e
    elif w.score_mode == "exact_mass":
        per_read = w.n_tokens * d * e + k * L * d * e + unread * 2 * d * e
    elif w.score_mode == "box":
        per_read = 2 * nb * d * e + unread * 2 * d * e + k * L * 2 * d * e
    elif w.score_mode == "proxy_error":  # mean and variance tokens of every block
        per_read = 2 * nb * d * e + unread * d * e + k * L * 2 * d * e
    elif w.score_mode == "cobs2_fp4":  # mean key, four fp32 scales and FP4 codes of every block
        per_read = nb * (2 * d + 16 + 4 * d // 2) + unread * d * e + k * L * 2 * d * e
    elif w.score_mode == "cobs2_sub":  # mean key and four padded subspace factors of every block
        sps = -(-w.sub_dim // 8) * 8
        per_read = nb * (d + 4 * sps) * e + unread * d * e + k * L * 2 * d * e
    elif w.score_mode == "cobs2_sub_fp4":  # mean key, four scales and four rows of FP4 codes of every block
        spf = -(-w.sub_dim // 32) * 32
        per_read = nb * (2 * d + 16 + 2 * spf) + unread * d * e + k * L * 2 * d * e
    else:  # second-order: the mean key and four eigenvector rows of every block
        per_read = 5 * nb * d * e + unread * d * e + k * L * 2 * d * e
    per_read += m * (2 * d * e + 8) + G * d * e
    per_write = G * (d + 1) * 4
    pairs = w.batch * w.n_kv_heads
    basis = w.n_kv_heads * d * w.sub_dim * 4 if w.score_mode.startswith("cobs2_sub") else 0  # U, once per step
    return pairs * per_read + basis, pairs * per_write


def graph_windows(g, steps, nwin):
    """ms per step of `nwin` windows, each one replay of a graph of `steps` launches.  A GPU
    sleep is queued before each window's start event, so the host has submitted the replay
    before the GPU reaches it: the window holds the launches' GPU time only."""
    import torch

    out = []
    for _ in range(nwin):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(200_000)  # about 0.1 ms at the GPU clock
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / steps)
    return out


def timed(fn, reps):
    """ms of `reps` eager calls of fn(r), HIP events around the loop."""
    import torch

    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for r in range(reps):
        fn(r)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def capture(fns, steps, nwin, warm):
    """One HIP graph per named route holding exactly `steps` launches of fn(i); each is replayed
    in `nwin` timed windows.  Returns {name: [ms per step of each window]}."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the capture stream
        for i in range(warm):
            for fn in fns.values():
                fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graphs = {}
    for name, fn in fns.items():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(i)
        graphs[name] = g
    for g in graphs.values():
        g.replay()
    torch.cuda.synchronize()
    return {name: graph_windows(g, steps, nwin) for name, g in graphs.items()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the selective decode path has no "
              "multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.counters:
        from coreset_softmax_attention_amd import workloads as W

        name = args.workload or W.HEADLINE
        counters_to_traffic(*args.counters, args.traffic or default_traffic_path(name), name)
        return

    import torch

    from coreset_softmax_attention_amd import csa
    from coreset_softmax_attention_amd import workloads as W

    if not os.path.exists(csa.library_path()):
        from coreset_softmax_attention_amd import build_lib

        build_lib.build()
    w = W.WORKLOADS[args.workload or W.HEADLINE]
    if w.score_mode == "cluster":
        cluster_main(args, w)
        return
    t0 = time.time()
    data = W.generate(w)
    print(f"[bench] generated {w.name} in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    NL = max(1, args.layers)
    q = csa.to_device(data["q"], dev)
    K0, V0 = csa.to_device(data["K"], dev), csa.to_device(data["V"], dev)
    tok_idx = csa.to_device(data["tok_idx"], dev) if w.coreset else None
    tok_logw = csa.to_device(data["tok_logw"], dev) if w.coreset else None
    m = w.coreset
    del data

    # prefill-time summaries of layer 0 (timed for information), then the other layers
    Kbar0, Vbar0 = csa.kv_summary_build(K0, V0, w.block_size)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    csa.kv_summary_build(K0, V0, w.block_size, Kbar0, Vbar0)
    e1.record()
    torch.cuda.synchronize()
    summary_ms = e0.elapsed_time(e1)
    box = w.score_mode in ("box", "cobs2", "proxy_error", "cobs2_fp4", "cobs2_sub", "cobs2_sub_fp4")  # extra summaries
    Kbox0 = None
    extra_ms = None
    Usub = None
    sub_fp4 = w.score_mode == "cobs2_sub_fp4"
    if w.score_mode.startswith("cobs2_sub"):  # the query basis of each KV head, from the seeded prefill queries
        sys.path.insert(0, os.path.join(HERE, "tests"))
        import qgc_inputs as QI

        Usub = torch.from_numpy(QI.pooled_query_basis(W.prefill_queries(w, 256), w.sub_dim)).to(dev)
    if box:
        build = {"box": csa.kv_box_build, "cobs2": csa.kv_cov_build, "proxy_error": csa.kv_var_build,
                 "cobs2_fp4": csa.kv_cov4_build,
                 "cobs2_sub": lambda K, L, out=None: csa.kv_cov_sub_build(K, Usub, L, out),
                 "cobs2_sub_fp4": lambda K, L, out=None: csa.kv_cov_sub_build(K, Usub, L, out, fp4=True)}[w.score_mode]
        Kbox0 = build(K0, w.block_size)
        torch.cuda.synchronize()
        e0.record()
        build(K0, w.block_size, Kbox0)
        e1.record()
        torch.cuda.synchronize()
        extra_ms = e0.elapsed_time(e1)
    layers = [(K0, V0, Kbar0, Vbar0, Kbox0)]
    for _ in range(NL - 1):
        layers.append(tuple(None if x is None else x.clone() for x in layers[0]))
    torch.cuda.synchronize()

    shape = csa.make_shape(q, K0, w.block_size)
    B, Hq, Hkv, nb = w.batch, w.n_q_heads, w.n_kv_heads, w.n_blocks
    scores = torch.empty((B, Hkv, nb), dtype=torch.float32, device=dev)
    sel = torch.empty((B, Hkv, min(w.k, nb)), dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    mode_entry = {"summary": csa.CSA_WS_BLOCK_SCORE_SUMMARY, "exact_mass": csa.CSA_WS_BLOCK_SCORE_EXACT_MASS,
                  "box": csa.CSA_WS_BLOCK_SCORE_BOX, "cobs2": csa.CSA_WS_BLOCK_SCORE_COBS2,
                  "proxy_error": csa.CSA_WS_BLOCK_SCORE_PROXY_ERROR,
                  "cobs2_fp4": csa.CSA_WS_BLOCK_SCORE_COBS2_FP4,
                  "cobs2_sub": csa.CSA_WS_BLOCK_SCORE_COBS2_SUB,
                  "cobs2_sub_fp4": csa.CSA_WS_BLOCK_SCORE_COBS2_SUB}[w.score_mode]
    ws_score = torch.empty(max(1, csa.workspace_size(shape, mode_entry)), dtype=torch.uint8, device=dev)
    ws_attn = torch.empty(max(1, csa.workspace_size(shape, csa.CSA_WS_SPARSE_DECODE_ATTN, w.k, m)),
                          dtype=torch.uint8, device=dev)
    ws_step = torch.empty(max(1, csa.workspace_size(shape, csa.CSA_WS_SELECTIVE_DECODE_STEP, w.k, m)),
                          dtype=torch.uint8, device=dev)

    def score_select(layer):
        K, V, Kbar, Vbar, Kbox = layer
        keys = Kbar if w.score_mode == "summary" else K if w.score_mode == "exact_mass" else Kbox
        if w.score_mode.startswith("cobs2_sub"):
            csa.block_score_cobs2_sub(q, keys, Usub, w.block_size, w.n_tokens, scores=scores, ws=ws_score, fp4=sub_fp4)
        else:
            csa.block_score(q, keys, w.score_mode, w.block_size, n_tokens=w.n_tokens, scores=scores, ws=ws_score)
        csa.topk_select(scores, w.k, sel=sel)

    def attend(layer):
        K, V, Kbar, Vbar, _ = layer
        csa.sparse_decode_attn(q, K, V, Kbar, Vbar, sel, w.block_size, proxies=w.proxies, tok_idx=tok_idx,
                               tok_logw=tok_logw, out=out, lse=lse, ws=ws_attn)

    def modular(i):
        score_select(layers[i % NL])
        attend(layers[i % NL])

    def step(i):
        if box:  # box and second-order scores need their summaries: the three entry points in turn
            modular(i)
            return
        K, V, Kbar, Vbar, _ = layers[i % NL]
        csa.selective_decode_step(q, K, V, Kbar, Vbar, w.k, w.block_size, mode=w.score_mode, proxies=w.proxies,
                                  tok_idx=tok_idx, tok_logw=tok_logw, out=out, lse=lse, ws=ws_step)

    # eager
    for i in range(args.warmup):
        step(i)
        modular(i)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    eager_ms = timed(step, args.steps) / args.steps
    wall = time.perf_counter() - wall0
    eager_modular_ms = timed(modular, args.steps) / args.steps

    graph_ms = attn_ms = score_ms = modular_ms = None
    windows = None
    if not args.no_graph:
        # one graph per route holding exactly K launches (layers cycled); each timed window
        # replays it once, so a window times exactly K steps
        windows = capture({"step": step, "modular": modular, "score": lambda i: score_select(layers[i % NL]),
                           "attn": lambda i: attend(layers[i % NL])}, args.steps, args.windows, NL)
        per = {name: float(np.median(v)) for name, v in windows.items()}
        graph_ms, modular_ms, score_ms, attn_ms = per["step"], per["modular"], per["score"], per["attn"]
    else:
        attn_ms = timed(lambda r: attend(layers[r % NL]), args.steps) / args.steps

    t_step = graph_ms if graph_ms is not None else eager_ms
    srd, swr = step_bytes(w, m)
    step_achieved = (srd + swr) / (t_step * 1e-3) / 1e9
    rd, wr = algorithmic_bytes(w, m)
    achieved = (rd + wr) / (attn_ms * 1e-3) / 1e9
    traffic = load_traffic(args.traffic or default_traffic_path(w.name))

    dense_ms = None
    if not args.no_dense:
        ws_dense = torch.empty(max(1, csa.workspace_size(shape, csa.CSA_WS_DENSE_DECODE_ATTN)), dtype=torch.uint8,
                               device=dev)
        dout, dlse = torch.empty_like(out), torch.empty_like(lse)

        def dense(r):
            K, V = layers[r % NL][:2]
            csa.dense_decode_attn(q, K, V, out=dout, lse=dlse, ws=ws_dense)

        dense(0)
        dense_ms = timed(dense, 2 * NL) / (2 * NL)

    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_seconds)

    result = {
        "metric": "selective decode attn: queries/s + achieved HBM GB/s, B=32, 32K ctx, 1% read",
        "value": B / (t_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "timing_detail": timing_detail(args, windows),
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
            "weighted_tokens": m, "layers_cycled": NL,
            "timing": "HIP graph of the decode step replayed" if graph_ms is not None else "eager",
            "entry_point": "block_score + topk_select + sparse_decode_attn" if box else "selective_decode_step",
        },
        "achieved_hbm_gb_s": step_achieved,
        "head_queries_per_s": B * Hq / (t_step * 1e-3),
        "eager_ms_per_step": eager_ms,
        "eager_wall_s": wall,
        "modular_ms_per_step": {"graph": modular_ms, "eager": eager_modular_ms},
        "modular_breakdown_us": {"block_score+topk_select": score_ms * 1e3 if score_ms else None,
                                 "sparse_decode_attn": attn_ms * 1e3},
        "kv_summary_build_ms": summary_ms,
        **({f"kv_{ {'box': 'box', 'cobs2': 'cov', 'proxy_error': 'var', 'cobs2_fp4': 'cov4', 'cobs2_sub': 'cov_sub', 'cobs2_sub_fp4': 'cov_sub4'}[w.score_mode]}_build_ms": extra_ms}
           if extra_ms is not None else {}),
        "dense_decode_attn_ms": dense_ms,
        "step_vs_dense_speedup": (dense_ms / t_step) if dense_ms else None,
        "roofline": {
            "kernel": "block_score + topk_select + sparse_decode_attn (three kernels)" if box
                      else step_kernels(w),
            "bound": "hbm",
            "achieved": step_achieved,
            "peak": 8000.0,
            "unit": "GB/s",
            "frac": step_achieved / 8000.0,
            "traffic": (three_call_traffic(traffic) if box else
                        traffic.get("decode_step") if isinstance(traffic, dict) else None),
            "algorithmic_bytes": srd + swr,
        },
        "roofline_sparse_decode_attn": {
            "kernel": "sparse_decode_attn (attn_mfma_kernel)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": 8000.0,
            "unit": "GB/s",
            "frac": achieved / 8000.0,
            "traffic": traffic.get("sparse_decode_attn") if isinstance(traffic, dict) else None,
            "algorithmic_bytes": rd + wr,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def cluster_bytes(w, sizes, sel):
    """Bytes the cluster decode step must move (reads, writes), and those of its attention
    kernel alone, from the selection actually made.  The step: every mean key once (it ranks
    the clusters and gives the proxy logits), the cluster ranges, the mean values of the
    unread non-empty clusters, the exact key/value rows of the selected clusters, the queries,
    the selection, the outputs with their log-normalisers.  The attention kernel: the mean key
    and value of each unread non-empty cluster, the exact rows, the ranges, the queries and
    selection, the outputs."""
    e, d, G, C = w.elem_bytes, w.head_dim, w.group, w.qgc
    pairs = w.batch * w.n_kv_heads
    sizes = sizes.reshape(pairs, C).astype(np.int64)
    sel = sel.reshape(pairs, -1).astype(np.int64)
    exact = int(np.take_along_axis(sizes, sel, axis=1).sum())
    unread = int((sizes > 0).sum()) - int((np.take_along_axis(sizes, sel, axis=1) > 0).sum())
    row = d * e
    common = pairs * ((C + 1) * 4 + G * row + 4 * sel.shape[1]) + exact * 2 * row
    writes = pairs * G * (d + 1) * 4
    step_rd = common + pairs * C * row + unread * row
    attn_rd = common + unread * 2 * row
    return {"step": (step_rd, writes), "attn": (attn_rd, writes), "exact_tokens": int(exact),
            "unread_clusters": unread}


def cluster_main(args, w):
    """The decode step over query-guided clusters (cluster_decode_step: cluster scores, top-k
    and attention) over a cache clustered once beforehand (kv_cluster_build, timed once for
    information), beside the three entry points in turn.  Same timing scheme as the block
    path."""
    import torch

    sys.path.insert(0, os.path.join(HERE, "tests"))
    import qgc_inputs as QI
    from coreset_softmax_attention_amd import csa
    from coreset_softmax_attention_amd import workloads as W

    t0 = time.time()
    data = W.generate(w)
    U = QI.query_basis(W.prefill_queries(w, 256), w.qgc_rank)
    seeds = QI.seed_tokens(w.batch, w.n_kv_heads, w.n_tokens, w.qgc)
    print(f"[bench] generated {w.name} in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    NL = max(1, args.layers)
    q = csa.to_device(data["q"], dev)
    K0, V0 = csa.to_device(data["K"], dev), csa.to_device(data["V"], dev)
    Ud, seedd = torch.from_numpy(U).to(dev), torch.from_numpy(seeds).to(dev)
    del data
    built = csa.kv_cluster_build(K0, V0, Ud, seedd, w.qgc_iters)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    csa.kv_cluster_build(K0, V0, Ud, seedd, w.qgc_iters, out=built)
    e1.record()
    torch.cuda.synchronize()
    build_ms = e0.elapsed_time(e1)
    del K0, V0
    layer0 = (built["Kg"], built["Vg"], built["Kc"], built["Vc"], built["offsets"])
    layers = [layer0] + [tuple(x.clone() for x in layer0) for _ in range(NL - 1)]
    torch.cuda.synchronize()

    B, Hq, Hkv, C = w.batch, w.n_q_heads, w.n_kv_heads, w.qgc
    shape = csa.make_shape(q, layer0[0], w.n_tokens)
    scores = torch.empty((B, Hkv, C), dtype=torch.float32, device=dev)
    sel = torch.empty((B, Hkv, min(w.k, C)), dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, csa.workspace_size(shape, csa.CSA_WS_CLUSTER_SCORE, C, 0)), dtype=torch.uint8,
                     device=dev)
    ws_step = torch.empty(max(1, csa.workspace_size(shape, csa.CSA_WS_CLUSTER_DECODE_STEP, w.k, C)),
                          dtype=torch.uint8, device=dev)

    def score_select(i):
        Kg, Vg, Kc, Vc, offs = layers[i % NL]
        csa.cluster_score(q, Kc, offs, w.n_tokens, scores=scores, ws=ws)
        csa.topk_select(scores, w.k, sel=sel)

    def attend(i):
        Kg, Vg, Kc, Vc, offs = layers[i % NL]
        csa.cluster_decode_attn(q, Kg, Vg, Kc, Vc, offs, sel, proxies=w.proxies, out=out, lse=lse)

    def modular(i):
        score_select(i)
        attend(i)

    def step(i):
        Kg, Vg, Kc, Vc, offs = layers[i % NL]
        csa.cluster_decode_step(q, Kg, Vg, Kc, Vc, offs, w.k, proxies=w.proxies, sel=sel, out=out, lse=lse,
                                ws=ws_step)

    for i in range(args.warmup):
        step(i)
        modular(i)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    eager_ms = timed(step, args.steps) / args.steps
    wall = time.perf_counter() - wall0
    windows = None
    modular_ms = None
    if not args.no_graph:
        windows = capture({"step": step, "modular": modular, "score": score_select, "attn": attend}, args.steps,
                          args.windows, NL)
        per = {name: float(np.median(v)) for name, v in windows.items()}
        t_step, modular_ms, score_ms, attn_ms = per["step"], per["modular"], per["score"], per["attn"]
    else:
        t_step, score_ms = eager_ms, None
        attn_ms = timed(attend, args.steps) / args.steps
    step(0)
    torch.cuda.synchronize()
    sizes = torch.diff(layer0[4], dim=-1).cpu().numpy()
    by = cluster_bytes(w, sizes, sel.cpu().numpy())
    step_achieved = sum(by["step"]) / (t_step * 1e-3) / 1e9
    attn_achieved = sum(by["attn"]) / (attn_ms * 1e-3) / 1e9
    traffic = load_traffic(args.traffic or default_traffic_path(w.name))
    cpu = None if args.no_cpu_baseline else cluster_cpu_baseline(w, args.cpu_seconds)
    result = {
        "metric": "selective decode attn: queries/s + achieved HBM GB/s, B=32, 32K ctx, 1% read",
        "value": B / (t_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "timing_detail": timing_detail(args, windows),
        "ms_per_step": t_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded generator; no dataset or weights)",
        "config": {
            "workload": w.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": w.head_dim,
            "context": w.n_tokens, "clusters": C, "cluster_rank": w.qgc_rank, "cluster_rounds": w.qgc_iters,
            "k_clusters": w.k, "exact_read_fraction": by["exact_tokens"] / (B * Hkv * w.n_tokens),
            "proxies": w.proxies, "layers_cycled": NL,
            "timing": "HIP graph of the decode step replayed" if windows else "eager",
            "entry_point": "cluster_decode_step",
        },
        "achieved_hbm_gb_s": step_achieved,
        "eager_ms_per_step": eager_ms,
        "eager_wall_s": wall,
        "modular_ms_per_step": modular_ms,
        "modular_breakdown_us": {"cluster_score+topk_select": score_ms * 1e3 if score_ms else None,
                                 "cluster_decode_attn": attn_ms * 1e3},
        "kv_cluster_build_ms": build_ms,
        "roofline": {
            "kernel": cluster_step_kernels(w),
            "bound": "hbm",
            "achieved": step_achieved,
            "peak": 8000.0,
            "unit": "GB/s",
            "frac": step_achieved / 8000.0,
            "traffic": traffic.get("decode_step") if isinstance(traffic, dict) else None,
            "algorithmic_bytes": sum(by["step"]),
        },
        "roofline_cluster_decode_attn": {
            "kernel": "cluster_decode_attn (cluster_attn_kernel)",
            "bound": "hbm",
            "achieved": attn_achieved,
            "peak": 8000.0,
            "unit": "GB/s",
            "frac": attn_achieved / 8000.0,
            "traffic": traffic.get("cluster_decode_attn") if isinstance(traffic, dict) else None,
            "algorithmic_bytes": sum(by["attn"]),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def cluster_cpu_baseline(w, budget_s):
    """The fp64 oracle's cluster decode step (cluster scores, top-k, attention) on the host cores
    for the first few sequences; their clustering (prefill state) is built before timing."""
    sys.path.insert(0, HERE)
    sys.path.insert(0, os.path.join(HERE, "tests"))
    import qgc_inputs as QI
    from coreset_softmax_attention_amd import workloads as W
    from oracle import oracle as O

    nseq = min(4, w.batch)
    sub = W.generate(w, batches=range(nseq))
    U = QI.query_basis(W.prefill_queries(w, 256, batches=range(nseq)), w.qgc_rank)
    seeds = QI.seed_tokens(nseq, w.n_kv_heads, w.n_tokens, w.qgc)
    shp = O.Shape(nseq, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_tokens, w.block_size, w.dtype)
    cl = O.cluster_build(shp, sub["K"], sub["V"], U, seeds, w.qgc_iters)  # cache state, not timed
    reps, t0 = 0, time.perf_counter()
    while True:
        score = O.cluster_score(shp, sub["q"], cl["Kc"], cl["offsets"])
        sel, _ = O.topk_select(score, w.k)
        O.cluster_attend(shp, sub["q"], sub["K"], sub["V"], cl["Kc"], cl["Vc"], cl["order"], cl["offsets"], sel,
                         w.proxies)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 100000:
            break
    cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    return {"value": nseq * reps / el, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} repetitions of the cluster decode step for the first {nseq} of {w.batch} sequences "
                      f"({el:.1f} s, fp64, OpenMP over query heads)", "cpu": cpu_model()}


def timing_detail(args, windows):
    """What was timed: windows of exactly `steps` launches, median reported."""
    if windows is None:
        return {"mode": "eager", "timed_launches": args.steps, "windows": 1}
    v = sorted(windows["step"])
    pick = lambda f: v[min(len(v) - 1, int(round(f * (len(v) - 1))))]
    return {"mode": "HIP graph of exactly `steps` launches, one replay per window, median window reported",
            "timed_launches_per_window": args.steps, "windows": len(v), "timed_launches": args.steps * len(v),
            "step_us": {"median": 1e3 * pick(0.5), "p10": 1e3 * pick(0.1), "p90": 1e3 * pick(0.9),
                        "min": 1e3 * v[0], "max": 1e3 * v[-1]}}


def cpu_model():
    """CPU model string with family / model / stepping, and the logical CPUs in this process's affinity."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (x.strip() for x in line.split(":", 1))
                if k in ("model name", "cpu family", "model", "stepping", "vendor_id") and k not in info:
                    info[k] = v
    except OSError:
        pass
    return (f"{info.get('model name', '?')} ({info.get('vendor_id', '?')} family {info.get('cpu family', '?')} "
            f"model {info.get('model', '?')} stepping {info.get('stepping', '?')}), "
            f"{len(os.sched_getaffinity(0))} logical CPUs in the process affinity")


def cpu_baseline(w, budget_s):
    """The fp64 oracle's decode step (block score, top-k, attention) on the host cores, on a
    bounded sample of the same workload: the first few sequences of the batch."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from coreset_softmax_attention_amd import workloads as W
    from oracle import oracle as O

    nseq = min(4, w.batch)
    sub = W.generate(w, batches=range(nseq))
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
        if el >= budget_s or reps >= 100000:
            break
    cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    return {"value": nseq * reps / el, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} repetitions of the decode step for the first {nseq} of {w.batch} sequences "
                      f"({el:.1f} s, fp64, OpenMP over KV heads)", "cpu": cpu_model()}


if __name__ == "__main__":
    main()
