"""Seeded synthetic decode workloads.

This module holds only the input recipe: random draws, their rounding to the
storage type, and the shapes.  It contains no step of the attention method, so
the HIP path and the fp64 oracle can both consume its arrays.

Every stream is a NumPy PCG64 generator seeded by a SeedSequence of
(workload seed, batch, KV head) for keys/values and (workload seed, batch,
query head, 1) for queries, so a stream does not depend on which other streams
are drawn, and a subset of the batch can be generated on its own.

Recipes (where a configuration text is open, the plainest reading is taken):

* tiny_f32_d64 -- B=1, one query and one KV head, d=64, n=1024, binary32.
  K, V ~ N(0, 1); q = 2 N(0, 1); 8 distinct heavy-hitter positions drawn
  uniformly, whose keys are 3 q/|q| + N(0, 0.1^2).  L=16, k=8.
* llama3_8b_layer_b1 / llama3_8b_layer_b32 -- Hq=32, Hkv=8, d=128, n=32768,
  bfloat16.  Per (b, KV head): 64 centres ~ N(0, I), 512 keys per centre at
  centre + 0.3 N(0, I), token order permuted; V ~ N(0, 1).  Query head h draws
  a centre of its KV head uniformly and adds 0.5 N(0, I).  L=64, k=5 (1 % of
  the tokens read exactly), summary score, proxies for every other block.
* exact_mass_mha_b8 / exact_mass_gqa_b8 -- B=8, Hq=32, Hkv=32 or 8, keys and
  queries as above; L=64, k=16, exact-mass score, no proxies.
* weighted_coreset_128k -- B=4, Hq=28, Hkv=4, n=131072, keys as above with
  2048 keys per centre; L=64, k=8, summary score, proxies; 2048 coreset
  indices per KV head drawn uniformly without replacement, w = exp(N(0, 1))
  rescaled in fp64 to sum n, log-weights stored as binary32.

Draws are made in binary32 (keys: centre + 0.3 noise computed in binary32) and
rounded to bfloat16 with round-to-nearest-even on the bit pattern.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_tokens: int
    block_size: int
    dtype: str  # "f32" or "bf16"
    k: int  # blocks read exactly per KV head
    score_mode: str  # "summary", "exact_mass", "box", "cobs2", "cobs2_fp4", "cobs2_sub", "cobs2_sub_fp4", "proxy_error" or "cluster"
    proxies: bool  # one count-aware proxy per unread block
    keys: str  # "heavy_hitters" or "clusters"
    n_clusters: int = 64
    coreset: int = 0  # weighted tokens per KV head
    description: str = ""
    qgc: int = 0  # query-guided clusters per KV head (score_mode "cluster"), 0 = blocks
    qgc_iters: int = 8  # Lloyd rounds of the cluster build
    qgc_rank: int = 16  # dimensions of the projection the clusters are found in
    sub_dim: int = 0  # query-subspace dimension s of the "cobs2_sub" descriptors

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_blocks(self) -> int:
        return -(-self.n_tokens // self.block_size)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32_d64", 1000, 1, 1, 1, 64, 1024, 16, "f32", 8, "summary", True, "heavy_hitters",
                 description="single-head fp32 decode with 8 planted heavy hitters"),
        Workload("llama3_8b_layer_b1", 1001, 1, 32, 8, 128, 32768, 64, "bf16", 5, "summary", True, "clusters",
                 description="Llama-3.1-8B-shaped layer, one sequence, 1% read + proxies"),
        Workload("llama3_8b_layer_b32", 1002, 32, 32, 8, 128, 32768, 64, "bf16", 5, "summary", True, "clusters",
                 description="Llama-3.1-8B-shaped layer, batch 32, 32K context, 1% read + proxies"),
        Workload("g8_layer_b32", 1006, 32, 64, 8, 128, 32768, 64, "bf16", 5, "summary", True, "clusters",
                 description="the headline cache read by 64 query heads (G = 8, a 70B-class layer), batch 32, "
                             "32K context, 1% read + proxies"),
        Workload("exact_mass_mha_b8", 1003, 8, 32, 32, 128, 32768, 64, "bf16", 16, "exact_mass", False, "clusters",
                 description="exact block masses (MHA), values read for the top-16 blocks only"),
        Workload("exact_mass_gqa_b8", 1013, 8, 32, 8, 128, 32768, 64, "bf16", 16, "exact_mass", False, "clusters",
                 description="exact block masses (GQA G=4), values read for the top-16 blocks only"),
        Workload("weighted_coreset_128k", 1004, 4, 28, 4, 128, 131072, 64, "bf16", 8, "summary", True, "clusters",
                 coreset=2048,
                 description="128K context, G=7: top-8 blocks + 2048 weighted coreset tokens + proxies"),
        Workload("llama3_8b_layer_b32_box", 1002, 32, 32, 8, 128, 32768, 64, "bf16", 5, "box", True, "clusters",
                 description="the headline layer with blocks ranked by their min/max key box (Quest)"),
        Workload("llama3_8b_layer_b32_cobs2", 1002, 32, 32, 8, 128, 32768, 64, "bf16", 5, "cobs2", True,
                 "clusters", description="the headline layer with second-order (mean + rank-4 covariance) scores"),
        Workload("llama3_8b_layer_b32_cobs2_fp4", 1002, 32, 32, 8, 128, 32768, 64, "bf16", 5, "cobs2_fp4", True,
                 "clusters", description="the headline layer with second-order scores from FP4 (E2M1) eigenvectors"),
        Workload("llama3_8b_layer_b32_cobs2_sub", 1002, 32, 32, 8, 128, 32768, 64, "bf16", 5, "cobs2_sub", True,
                 "clusters", sub_dim=85,
                 description="the headline layer with second-order scores whose covariance is kept in an "
                             "85-dimensional query subspace (340 instead of 512 factor floats per block)"),
        Workload("llama3_8b_layer_b32_cobs2_sub_fp4", 1002, 32, 32, 8, 128, 32768, 64, "bf16", 5, "cobs2_sub_fp4",
                 True, "clusters", sub_dim=85,
                 description="the headline layer with second-order scores from 85-dimensional query-subspace "
                             "factors stored in FP4 (464 bytes per block)"),
        Workload("llama3_8b_layer_b32_err", 1002, 32, 32, 8, 128, 32768, 64, "bf16", 5, "proxy_error", True,
                 "clusters", description="the headline layer with exact reads spent on the largest estimated "
                                         "proxy errors (mean and variance tokens)"),
        Workload("llama3_8b_layer_b32_qgc", 1002, 32, 32, 8, 128, 32768, 64, "bf16", 5, "cluster", True,
                 "clusters", qgc=512, description="the headline layer with one proxy per query-guided cluster "
                                                  "(512 k-means clusters in the 16-dimensional query subspace) "
                                                  "and the tokens of the top-5 clusters read exactly"),
    ]
}

HEADLINE = "llama3_8b_layer_b32"


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 array -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(w: Workload, x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, np.float32) if w.dtype == "f32" else to_bf16_bits(x)


def _kv_rng(w: Workload, b: int, j: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, b, j])))


def _q_rng(w: Workload, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, b, h, 1])))


def _centres(w: Workload, rng: np.random.Generator) -> np.ndarray:
    return rng.standard_normal((w.n_clusters, w.head_dim), dtype=np.float32)


def _kv_stream(w: Workload, b: int, j: int):
    """Draw stream (b, j): returns K[b, j], V[b, j] and the coreset lists (or None)."""
    rng = _kv_rng(w, b, j)
    n, d = w.n_tokens, w.head_dim
    if w.keys == "clusters":
        centres = _centres(w, rng)
        per = n // w.n_clusters
        assert per * w.n_clusters == n, "token count must split evenly over the clusters"
        keys = rng.standard_normal((n, d), dtype=np.float32)
        keys *= np.float32(0.3)
        keys += np.repeat(centres, per, axis=0)
        perm = rng.permutation(n)
        k_bj = _store(w, keys[perm])
        del keys
        v_bj = _store(w, rng.standard_normal((n, d), dtype=np.float32))
    else:  # heavy_hitters: some key rows are replaced from the query stream
        k_bj = _store(w, rng.standard_normal((n, d)))
        v_bj = _store(w, rng.standard_normal((n, d)))
    idx = logw = None
    if w.coreset:
        idx = rng.choice(n, size=w.coreset, replace=False).astype(np.int32)
        wts = np.exp(rng.standard_normal(w.coreset))
        wts *= n / wts.sum()
        logw = np.log(wts).astype(np.float32)
    return k_bj, v_bj, idx, logw


def _q_stream(w: Workload, b: int, h: int):
    """Draw query head (b, h): returns q[b, h] and (positions, key rows) to plant, or None."""
    rng = _q_rng(w, b, h)
    if w.keys == "clusters":
        centres = _centres(w, _kv_rng(w, b, h // w.group))  # the first draws of the KV stream
        c = int(rng.integers(w.n_clusters))
        qv = centres[c] + np.float32(0.5) * rng.standard_normal(w.head_dim, dtype=np.float32)
        return _store(w, qv), None
    qv = 2.0 * rng.standard_normal(w.head_dim)
    pos = rng.choice(w.n_tokens, size=8, replace=False)
    hh = 3.0 * qv / np.linalg.norm(qv) + 0.1 * rng.standard_normal((8, w.head_dim))
    return _store(w, qv), (pos, _store(w, hh))


def generate(w: Workload, batches=None, threads: int | None = None) -> dict:
    """Draw the inputs of workload w for the given batch entries (default: all).

    Returns a dict with q [B', Hq, d], K, V [B', Hkv, n, d] (float32 or uint16
    bfloat16 bits) and, for coreset workloads, tok_idx int32 / tok_logw float32
    [B', Hkv, m].  B' = len(batches); entry i holds batch index batches[i]."""
    batches = list(range(w.batch)) if batches is None else list(batches)
    Bp = len(batches)
    st = np.float32 if w.dtype == "f32" else np.uint16
    K = np.empty((Bp, w.n_kv_heads, w.n_tokens, w.head_dim), st)
    V = np.empty_like(K)
    q = np.empty((Bp, w.n_q_heads, w.head_dim), st)
    tok_idx = np.empty((Bp, w.n_kv_heads, w.coreset), np.int32) if w.coreset else None
    tok_logw = np.empty((Bp, w.n_kv_heads, w.coreset), np.float32) if w.coreset else None

    def kv_job(t):
        i, b, j = t
        K[i, j], V[i, j], idx, logw = _kv_stream(w, b, j)
        if w.coreset:
            tok_idx[i, j], tok_logw[i, j] = idx, logw

    jobs = [(i, b, j) for i, b in enumerate(batches) for j in range(w.n_kv_heads)]
    with ThreadPoolExecutor(threads or min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(kv_job, jobs))
    # query streams after the key streams: planted heavy hitters overwrite key rows
    for i, b in enumerate(batches):
        for h in range(w.n_q_heads):
            q[i, h], plant = _q_stream(w, b, h)
            if plant is not None:
                pos, rows = plant
                K[i, h // w.group, pos] = rows
    out = {"q": q, "K": K, "V": V}
    if w.coreset:
        out["tok_idx"], out["tok_logw"] = tok_idx, tok_logw
    return out


def prefill_queries(w: Workload, count: int, batches=None) -> np.ndarray:
    """Queries seen during prefill, [B', Hkv, count, d] float64: for each KV head, `count` draws
    of the decode-query recipe (a centre of the KV head's key clusters + 0.5 N(0, I)) from a
    stream of their own (seed, b, KV head, 2).  Random data only: what a caller derives from
    them (the query basis of the cluster build) is computed by the caller."""
    batches = list(range(w.batch)) if batches is None else list(batches)
    out = np.empty((len(batches), w.n_kv_heads, count, w.head_dim), np.float64)
    for i, b in enumerate(batches):
        for j in range(w.n_kv_heads):
            centres = _centres(w, _kv_rng(w, b, j)).astype(np.float64)
            rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, b, j, 2])))
            pick = rng.integers(w.n_clusters, size=count)
            out[i, j] = centres[pick] + 0.5 * rng.standard_normal((count, w.head_dim))
    return out


def scaled_down(w: Workload, batch=None, n_tokens=None, n_kv_heads=None) -> Workload:
    """Same recipe at a smaller size (for tests that the oracle must finish quickly)."""
    kw = {}
    if batch is not None:
        kw["batch"] = batch
    if n_tokens is not None:
        kw["n_tokens"] = n_tokens
    if n_kv_heads is not None:
        kw["n_q_heads"] = w.group * n_kv_heads
        kw["n_kv_heads"] = n_kv_heads
    return replace(w, name=w.name + "_scaled", **kw)
