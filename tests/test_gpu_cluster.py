"""Parity of the query-guided cluster path (kv_cluster_build, cluster_score, topk_select,
cluster_decode_attn through the C-ABI) with the fp64 oracle on the same seeded inputs.

Bars: the build (assignments, order, ranges, the gathered cache, the cluster means) bit-exact --
both sides evaluate the same fp64 operations in the same order; scores, selections, outputs and
lse as in the block path's parity tests (score bound 1e-4 + 1e-5 |s|, near-tied selection rows
only may differ, output rows 2e-3 relative, lse 1e-3 for bfloat16).
"""
import numpy as np
import pytest
import torch

import qgc_inputs as QI
from coreset_softmax_attention_amd import csa
from coreset_softmax_attention_amd import workloads as W
from oracle import oracle as O
from test_gpu_parity import assert_out, assert_scores, assert_selection, bits, dev, host

pytestmark = pytest.mark.gpu


def case(name, seed, B, Hkv, G, d, n, C, r, dtype="bf16", k=3, iters=4):
    w = W.Workload(name, seed, B, Hkv * G, Hkv, d, n, 64, dtype, k, "cluster", True, "clusters", n_clusters=16,
                   qgc=C, qgc_rank=r, qgc_iters=iters)
    return w


CASES = [
    case("g4_d128_r16", 3001, 2, 2, 4, 128, 3008, 64, 16),
    case("g1_d64_r4", 3002, 1, 3, 1, 64, 2048, 40, 4, k=2, iters=3),
    case("g8_d128_r32", 3003, 1, 2, 8, 128, 4096, 200, 32, k=6, iters=2),
    case("g7_d128_r8", 3004, 1, 1, 7, 128, 1984, 33, 8, k=4, iters=5),
    case("g2_d64_f32", 3005, 1, 2, 2, 64, 1024, 24, 8, dtype="f32", iters=3),
    case("g3_d128_iters0", 3006, 2, 1, 3, 128, 1536, 48, 16, iters=0),
]


def inputs(w, seeds=None):
    data = W.generate(w)
    U = QI.query_basis(W.prefill_queries(w, 256), w.qgc_rank)
    if seeds is None:
        seeds = QI.seed_tokens(w.batch, w.n_kv_heads, w.n_tokens, w.qgc)
    return data, U, seeds


def oshape(w):
    return O.Shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_tokens, w.block_size, w.dtype)


def gpu_build(w, data, U, seeds):
    r = csa.kv_cluster_build(dev(data["K"]), dev(data["V"]), torch.from_numpy(np.ascontiguousarray(U)).cuda(),
                             torch.from_numpy(np.ascontiguousarray(seeds)).cuda(), w.qgc_iters)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in r.items()}


def compare_build(w, data, g, o, what):
    for name in ("assign", "order", "offsets"):
        assert np.array_equal(g[name], o[name]), f"{what}: {name} differs"
    for name in ("Kc", "Vc"):
        assert np.array_equal(bits(g[name]), bits(o[name])), f"{what}: {name} not bit-exact"
    gathered = lambda X: np.take_along_axis(X, o["order"][..., None].astype(np.int64), axis=2)
    assert np.array_equal(bits(g["Kg"]), bits(gathered(data["K"]))), f"{what}: Kg is not K in cluster order"
    assert np.array_equal(bits(g["Vg"]), bits(gathered(data["V"]))), f"{what}: Vg is not V in cluster order"


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_cluster_build_bit_exact(w):
    data, U, seeds = inputs(w)
    o = O.cluster_build(oshape(w), data["K"], data["V"], U, seeds, w.qgc_iters)
    compare_build(w, data, gpu_build(w, data, U, seeds), o, w.name)


def test_cluster_build_empty_clusters():
    """Repeated seeds and no update round: the higher of two equal centroids never wins a token
    (ties go to the lower index), so its cluster is empty -- empty ranges, zero means, -inf
    scores, no proxy."""
    w = case("empty", 3010, 1, 2, 4, 128, 2048, 32, 16, iters=0)
    seeds = QI.seed_tokens(1, 2, w.n_tokens, w.qgc)
    seeds[..., 5] = seeds[..., 4]
    seeds[..., 31] = seeds[..., 0]
    data, U, _ = inputs(w)
    o = O.cluster_build(oshape(w), data["K"], data["V"], U, seeds, w.qgc_iters)
    cnt = np.diff(o["offsets"], axis=-1)
    assert (cnt[..., 5] == 0).all() and (cnt[..., 31] == 0).all()
    g = gpu_build(w, data, U, seeds)
    compare_build(w, data, g, o, "empty clusters")
    check_decode(w, data, o, "empty clusters", k=4)


def check_decode(w, data, o, what, k=None, proxies_list=(True, False)):
    """Scores, selection and attention from the oracle's build (inputs of both sides)."""
    k = w.k if k is None else k
    shp = oshape(w)
    q = dev(data["q"])
    Kc, offs = dev(o["Kc"]), torch.from_numpy(o["offsets"]).cuda()
    scores = csa.cluster_score(q, Kc, offs, w.n_tokens)
    sel = csa.topk_select(scores, k)
    torch.cuda.synchronize()
    ref_score = O.cluster_score(shp, data["q"], o["Kc"], o["offsets"])
    ref_sel, margin = O.topk_select(ref_score, k)
    err = assert_scores(host(scores), ref_score, what)
    assert_selection(host(sel), ref_sel, ref_score, margin, what, err)
    if w.dtype != "bf16":
        with pytest.raises(csa.CsaError) as ei:
            csa.cluster_decode_attn(q, dev(o["Kc"]), dev(o["Vc"]), Kc, dev(o["Vc"]), offs,
                                    torch.from_numpy(ref_sel).cuda())
        assert ei.value.status == csa.CSA_ERR_UNSUPPORTED
        return
    Kg = np.take_along_axis(data["K"], o["order"][..., None].astype(np.int64), axis=2)
    Vg = np.take_along_axis(data["V"], o["order"][..., None].astype(np.int64), axis=2)
    Kgd, Vgd, Vcd = dev(Kg), dev(Vg), dev(o["Vc"])
    for proxies in proxies_list:
        out, lse = csa.cluster_decode_attn(q, Kgd, Vgd, Kc, Vcd, offs,
                                           torch.from_numpy(np.ascontiguousarray(ref_sel)).cuda(), proxies=proxies)
        torch.cuda.synchronize()
        ref_out, ref_lse = O.cluster_attend(shp, data["q"], data["K"], data["V"], o["Kc"], o["Vc"], o["order"],
                                            o["offsets"], ref_sel, proxies)
        assert_out(host(out), host(lse), ref_out, ref_lse, w.dtype, f"{what} proxies={proxies}")
        # the one-call step: the same scores and selection as the entry points in turn, and
        # the oracle's outputs for its selection
        so, sl, ss, ssel = csa.cluster_decode_step(q, Kgd, Vgd, Kc, Vcd, offs, k, proxies=proxies, want_scores=True,
                                                   want_sel=True)
        torch.cuda.synchronize()
        assert np.array_equal(bits(host(ss)), bits(host(scores))), f"{what}: step scores differ"
        assert np.array_equal(host(ssel), host(sel)), f"{what}: step selection differs"
        step_ref = (ref_out, ref_lse)
        if not np.array_equal(host(sel), ref_sel):  # near-tied rows chose otherwise: attend to the GPU's choice
            step_ref = O.cluster_attend(shp, data["q"], data["K"], data["V"], o["Kc"], o["Vc"], o["order"],
                                        o["offsets"], host(sel), proxies)
        assert_out(host(so), host(sl), *step_ref, w.dtype, f"{what} step proxies={proxies}")


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_cluster_decode_parity(w):
    data, U, seeds = inputs(w)
    o = O.cluster_build(oshape(w), data["K"], data["V"], U, seeds, w.qgc_iters)
    check_decode(w, data, o, w.name)


def test_cluster_decode_edges():
    """k = 0 (proxies only), k = C (every cluster read exactly: dense attention), one cluster."""
    w = case("edges", 3020, 1, 2, 4, 128, 2048, 24, 8, iters=2)
    data, U, seeds = inputs(w)
    shp = oshape(w)
    o = O.cluster_build(shp, data["K"], data["V"], U, seeds, w.qgc_iters)
    check_decode(w, data, o, "k=0", k=0, proxies_list=(True,))
    check_decode(w, data, o, "k=1", k=1)
    check_decode(w, data, o, "k=C", k=w.qgc)
    # every cluster exact equals dense attention over the cache
    Kg = np.take_along_axis(data["K"], o["order"][..., None].astype(np.int64), axis=2)
    Vg = np.take_along_axis(data["V"], o["order"][..., None].astype(np.int64), axis=2)
    sel = np.broadcast_to(np.arange(w.qgc, dtype=np.int32), (1, 2, w.qgc)).copy()
    out, lse = csa.cluster_decode_attn(dev(data["q"]), dev(Kg), dev(Vg), dev(o["Kc"]), dev(o["Vc"]),
                                       torch.from_numpy(o["offsets"]).cuda(), torch.from_numpy(sel).cuda())
    torch.cuda.synchronize()
    ref, ref_lse = O.dense_decode_attn(shp, data["q"], data["K"], data["V"])
    assert_out(host(out), host(lse), ref, ref_lse, "bf16", "all clusters vs dense")
    # a single cluster holding every token: its proxy alone is the mean value
    one = case("one", 3021, 1, 1, 2, 64, 512, 1, 4, iters=1)
    d1, U1, s1 = inputs(one)
    o1 = O.cluster_build(oshape(one), d1["K"], d1["V"], U1, s1, 1)
    check_decode(one, d1, o1, "C=1", k=1)
    check_decode(one, d1, o1, "C=1 proxy only", k=0, proxies_list=(True,))


# 32 or more KV heads, k <= 32, C <= 2048: cluster_decode_step runs as one kernel per KV head
STEP_CASES = [
    case("step_g4_d128", 3101, 8, 4, 4, 128, 1024, 48, 8, k=5, iters=2),
    case("step_g8_d64_k32", 3102, 4, 8, 8, 64, 768, 100, 4, k=32, iters=1),
    case("step_g1_c600", 3103, 16, 2, 1, 128, 2048, 600, 8, k=3, iters=1),
    case("step_g3_d128", 3104, 32, 1, 3, 128, 640, 37, 16, k=7, iters=2),
]


def fused_step_runs(w, data, o, k, proxies=True):
    """The one-kernel route leaves the workspace alone (the kernels in turn keep their scores
    and selection there when the caller passes no buffers for them)."""
    q, Kc, offs = dev(data["q"]), dev(o["Kc"]), torch.from_numpy(o["offsets"]).cuda()
    Kg = np.take_along_axis(data["K"], o["order"][..., None].astype(np.int64), axis=2)
    Vg = np.take_along_axis(data["V"], o["order"][..., None].astype(np.int64), axis=2)
    shape = csa.make_shape(q, dev(Kg), w.n_tokens, 0.0)
    need = csa.workspace_size(shape, csa.CSA_WS_CLUSTER_DECODE_STEP, k, w.qgc)
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")
    csa.cluster_decode_step(q, dev(Kg), dev(Vg), Kc, dev(o["Vc"]), offs, k, proxies=proxies, ws=ws)
    torch.cuda.synchronize()
    return bool((ws == 0xAB).all().item())


@pytest.mark.parametrize("w", STEP_CASES, ids=[c.name for c in STEP_CASES])
def test_cluster_step_one_kernel(w):
    data, U, seeds = inputs(w)
    o = O.cluster_build(oshape(w), data["K"], data["V"], U, seeds, w.qgc_iters)
    assert fused_step_runs(w, data, o, w.k), f"{w.name}: not the one-kernel route"
    check_decode(w, data, o, w.name)


def test_cluster_step_one_kernel_edges():
    """The one-kernel route with empty clusters (count term -inf: never a proxy, last in the
    ranking), k = 0 (proxies only) and k = C (every cluster exact: dense attention)."""
    w = case("step_edges", 3110, 8, 4, 2, 128, 1024, 24, 8, iters=0)
    seeds = QI.seed_tokens(w.batch, w.n_kv_heads, w.n_tokens, w.qgc)
    seeds[..., 7] = seeds[..., 3]
    seeds[..., 23] = seeds[..., 0]
    data, U, _ = inputs(w)
    o = O.cluster_build(oshape(w), data["K"], data["V"], U, seeds, w.qgc_iters)
    cnt = np.diff(o["offsets"], axis=-1)
    assert (cnt[..., 7] == 0).all() and (cnt[..., 23] == 0).all()
    for k in (0, 4, 22, 24):
        assert fused_step_runs(w, data, o, k), f"k={k}: not the one-kernel route"
    check_decode(w, data, o, "step empty clusters", k=4)
    check_decode(w, data, o, "step k=22 (with empty ones)", k=22)
    check_decode(w, data, o, "step k=0", k=0, proxies_list=(True,))
    check_decode(w, data, o, "step k=C", k=w.qgc)
    Kg = np.take_along_axis(data["K"], o["order"][..., None].astype(np.int64), axis=2)
    Vg = np.take_along_axis(data["V"], o["order"][..., None].astype(np.int64), axis=2)
    out, lse, _, _ = csa.cluster_decode_step(dev(data["q"]), dev(Kg), dev(Vg), dev(o["Kc"]), dev(o["Vc"]),
                                             torch.from_numpy(o["offsets"]).cuda(), w.qgc, proxies=False)
    torch.cuda.synchronize()
    ref, ref_lse = O.dense_decode_attn(oshape(w), data["q"], data["K"], data["V"])
    assert_out(host(out), host(lse), ref, ref_lse, "bf16", "one-kernel step, all clusters vs dense")


def test_cluster_index_checks_reject_what_the_oracle_rejects():
    w = case("checks", 3030, 1, 2, 2, 64, 1024, 16, 8, iters=1)
    data, U, seeds = inputs(w)
    o = O.cluster_build(oshape(w), data["K"], data["V"], U, seeds, 1)
    prev = csa.set_index_checks(True)
    try:
        bad = seeds.copy()
        bad[0, 1, 3] = w.n_tokens
        with pytest.raises(csa.CsaError) as ei:
            gpu_build(w, data, U, bad)
        assert ei.value.status == csa.CSA_ERR_INVALID_ARG
        with pytest.raises(Exception):
            O.cluster_build(oshape(w), data["K"], data["V"], U, bad, 1)
        Kc, Vc, offs = dev(o["Kc"]), dev(o["Vc"]), torch.from_numpy(o["offsets"]).cuda()
        for row in ([1, 1, 2], [0, 3, 16], [-1, 2, 3]):
            sel = torch.tensor([[row, [0, 1, 2]]], dtype=torch.int32).cuda()
            with pytest.raises(csa.CsaError) as ei:
                csa.cluster_decode_attn(dev(data["q"]), dev(data["K"]), dev(data["V"]), Kc, Vc, offs, sel)
            assert ei.value.status == csa.CSA_ERR_INVALID_ARG, row
    finally:
        csa.set_index_checks(prev)


# ---------------------------------------------------------------------------
# the headline layer with query-guided clusters, every (sequence, KV head)
# ---------------------------------------------------------------------------

def test_cluster_full_size_all_pairs():
    """32 sequences x 8 KV heads x 32768 tokens, 512 clusters in the 16-dimensional query
    subspace, 8 rounds: the GPU build, scores, top-5 and attention against the oracle on every
    (sequence, KV head)."""
    w = W.WORKLOADS["llama3_8b_layer_b32_qgc"]
    data, U, seeds = inputs(w)
    g = gpu_build(w, data, U, seeds)
    o = O.cluster_build(oshape(w), data["K"], data["V"], U, seeds, w.qgc_iters)
    compare_build(w, data, g, o, w.name)
    del g
    check_decode(w, data, o, w.name, proxies_list=(True,))
