"""Parity of the query-subspace second-order descriptors (kv_cov_sub_build) and scores
(block_score_cobs2_sub) with the fp64 oracle.

As for the full-space descriptors: the mean rows are bit-exact; the factors span the oracle's
top eigenspace of U^T Sigma_b U (sum_i xi_i xi_i^T within a relative Frobenius tolerance) on
every block where that space is unique; the padding is zero.  Scores: the GPU's against the
oracle's on the same stored descriptors, within the score bound (1e-4 + 1e-5 |s|); selection
bit-exact outside near-tied rows; end to end (each side building its own descriptors from the
keys), rows may select differently only where the oracle's margin is within what the
descriptor rounding can move.
"""
import numpy as np
import pytest
import torch

import qgc_inputs as QI
from coreset_softmax_attention_amd import csa
from coreset_softmax_attention_amd import workloads as W
from oracle import oracle as O
from test_gpu_parity import assert_out, assert_scores, assert_selection, bits, dev, host, oshape, rand_inputs

pytestmark = pytest.mark.gpu


def basis(w, s_dim, batches=None):
    return QI.pooled_query_basis(W.prefill_queries(w, 256, batches), s_dim)


def check_sub_descriptors(kc, K, U, shp, what, tol):
    """Mean rows bit for bit, zero padding, and the factors' eigenspace (see the module doc)."""
    s_dim, d, r = U.shape[-1], shp.head_dim, O.COBS_RANK
    sp = O.sub_padded(s_dim)
    Kbar_o, _ = O.kv_summary_build(shp, K, K)
    assert np.array_equal(bits(kc[..., :d]), bits(Kbar_o)), f"{what}: mean rows not bit-exact"
    fac = kc[..., d:].reshape(kc.shape[:3] + (r, sp))
    assert np.all(fac[..., s_dim:] == 0), f"{what}: padding not zero"
    xo = O.cov_sub_factors(shp, K, U)
    Kf = O.widen(shp, K)
    L, n = shp.block_size, shp.n_tokens
    checked = 0
    for b in range(kc.shape[0]):
        for j in range(kc.shape[1]):
            Uj = U[j].astype(np.float64)
            for blk in range(shp.n_blocks):
                X = Kf[b, j, blk * L:min(n, (blk + 1) * L)]
                Y = (X - X.mean(axis=0)) @ Uj
                mu = np.linalg.eigvalsh(Y.T @ Y / X.shape[0])[::-1] if X.shape[0] > 1 else np.zeros(r + 1)
                if len(mu) > r and mu[0] > 0 and mu[r - 1] > 1e-5 * mu[0] and (mu[r - 1] - mu[r]) < 1e-2 * mu[0]:
                    continue  # a 4th direction that is both weighty and not unique
                A = O.widen(shp, fac[b, j, blk, :, :s_dim])
                B = xo[b, j, blk]
                PA, PB = A.T @ A, B.T @ B
                assert np.linalg.norm(PA - PB) <= tol * max(np.linalg.norm(PB), 1e-30), \
                    f"{what}: block ({b},{j},{blk}) eigenspace differs"
                checked += 1
    assert checked >= 0.8 * kc.shape[0] * kc.shape[1] * shp.n_blocks, f"{what}: too few blocks checked"


CASES = [  # name, B, Hkv, G, d, n, L, s, dtype, tol
    ("bf16_d128_s85", 2, 2, 4, 128, 4096, 64, 85, "bf16", 2e-2),
    ("bf16_d128_s128", 1, 2, 4, 128, 2048, 64, 128, "bf16", 2e-2),
    ("bf16_d128_s20_ragged", 2, 1, 7, 128, 3000, 64, 20, "bf16", 2e-2),
    ("bf16_d64_s30_L32", 2, 2, 2, 64, 2048, 32, 30, "bf16", 2e-2),
    ("f32_d64_s9_L16", 1, 2, 1, 64, 700, 16, 9, "f32", 1e-4),
]


@pytest.mark.parametrize("name,B,Hkv,G,d,n,L,s_dim,dtype,tol", CASES, ids=[c[0] for c in CASES])
def test_sub_descriptors_match_oracle(name, B, Hkv, G, d, n, L, s_dim, dtype, tol):
    w = W.Workload(name, 4000 + n, B, G * Hkv, Hkv, d, n, L, dtype, 3, "cobs2_sub", True, "clusters", sub_dim=s_dim)
    data = rand_inputs(4000 + n + s_dim, B, G * Hkv, Hkv, d, n, dtype)
    U = basis(w, s_dim)
    kc = host(csa.kv_cov_sub_build(dev(data["K"]), torch.from_numpy(U).cuda(), L))
    torch.cuda.synchronize()
    check_sub_descriptors(kc, data["K"], U, oshape(w), name, tol)


def sub_case(w, data, U, k):
    q, K = dev(data["q"]), dev(data["K"])
    Ud = torch.from_numpy(U).cuda()
    Kcs = csa.kv_cov_sub_build(K, Ud, w.block_size)
    scores = csa.block_score_cobs2_sub(q, Kcs, Ud, w.block_size, w.n_tokens)
    sel = csa.topk_select(scores, k)
    torch.cuda.synchronize()
    return host(Kcs), host(scores), host(sel)


@pytest.mark.parametrize("name,B,Hkv,G,d,n,L,s_dim,dtype,tol", [c for c in CASES if c[8] == "bf16"],
                         ids=[c[0] for c in CASES if c[8] == "bf16"])
def test_sub_scores_and_selection(name, B, Hkv, G, d, n, L, s_dim, dtype, tol):
    w = W.Workload(name, 4100 + n, B, G * Hkv, Hkv, d, n, L, dtype, 5, "cobs2_sub", True, "clusters", sub_dim=s_dim)
    data = W.generate(w) if n % 64 == 0 else rand_inputs(4100 + n, B, G * Hkv, Hkv, d, n, dtype)
    U = basis(w, s_dim)
    kc, sc, sel = sub_case(w, data, U, w.k)
    shp = oshape(w)
    ref = O.group_score(shp, O.cobs2_sub_logits(shp, data["q"], kc, U))
    ref_sel, margin = O.topk_select(ref, w.k)
    err = assert_scores(sc, ref, name)
    assert_selection(sel, ref_sel, ref, margin, name, err)


def test_sub_score_of_full_dimension_equals_the_full_space_score():
    """s = d: the subspace scores of the GPU agree with its full-space second-order scores up to
    the descriptors' rounding (each from its own build), on the same keys."""
    w = W.scaled_down(W.WORKLOADS["llama3_8b_layer_b32_cobs2_sub"], batch=2, n_tokens=4096, n_kv_heads=2)
    data = W.generate(w)
    U = basis(w, 128)
    _, sc_sub, _ = sub_case(w, data, U, w.k)
    q, K = dev(data["q"]), dev(data["K"])
    sc_full = host(csa.block_score(q, csa.kv_cov_build(K, w.block_size), "cobs2", w.block_size, n_tokens=w.n_tokens))
    torch.cuda.synchronize()
    assert np.abs(sc_sub - sc_full).max() <= 2e-2 * (1 + np.abs(sc_full).max())


def test_sub_full_size_all_pairs():
    """The headline layer, s = 85: descriptors of sampled KV heads against the oracle's solve,
    and the scores and top-5 of every (sequence, KV head)."""
    w = W.WORKLOADS["llama3_8b_layer_b32_cobs2_sub"]
    data = W.generate(w)
    U = basis(w, w.sub_dim)
    kc, sc, sel = sub_case(w, data, U, w.k)
    shp = oshape(w)
    ref = O.group_score(shp, O.cobs2_sub_logits(shp, data["q"], kc, U))
    ref_sel, margin = O.topk_select(ref, w.k)
    err = assert_scores(sc, ref, w.name)
    assert_selection(sel, ref_sel, ref, margin, w.name, err)
    for b, j in ((0, 0), (17, 3), (31, 7)):
        check_sub_descriptors(kc[b:b + 1, j:j + 1], data["K"][b:b + 1, j:j + 1], U[j:j + 1], oshape(w, B=1, Hkv=1),
                              f"{w.name} ({b},{j})", 2e-2)


def test_sub_end_to_end_selection_agreement():
    """Each side builds its own descriptors from the keys (GPU fp32 solve, oracle fp64) and
    ranks with them: a row may select differently only where the oracle's k-th margin is small
    against what the bfloat16 rounding of the factors can move a score, and few rows do."""
    w = W.scaled_down(W.WORKLOADS["llama3_8b_layer_b32_cobs2_sub"], batch=4, n_tokens=8192, n_kv_heads=4)
    data = W.generate(w)
    U = basis(w, w.sub_dim)
    _, sc, sel = sub_case(w, data, U, w.k)
    shp = oshape(w)
    ko = O.cov_sub_build(shp, data["K"], U)
    ref = O.group_score(shp, O.cobs2_sub_logits(shp, data["q"], ko, U))
    ref_sel, margin = O.topk_select(ref, w.k)
    sel, ref_sel, margin = sel.reshape(-1, w.k), ref_sel.reshape(-1, w.k), np.asarray(margin).reshape(-1)
    pert = np.abs(sc - ref).reshape(-1, sc.shape[-1]).max(axis=1)
    differ = [r for r in range(sel.shape[0]) if not np.array_equal(sel[r], ref_sel[r])]
    for r in differ:
        assert margin[r] <= 2 * pert[r] + 2e-4, f"row {r}: margin {margin[r]:.3e} against score moves {pert[r]:.3e}"
    assert len(differ) <= sel.shape[0] // 4
    print(f"query-subspace ranking end to end (descriptors built on each side): "
          f"{sel.shape[0] - len(differ)} of {sel.shape[0]} rows select the same blocks")


# ---------------------------------------------------------------------------
# FP4 factors
# ---------------------------------------------------------------------------

FP4_CASES = [c for c in CASES if c[8] == "bf16"]


@pytest.mark.parametrize("name,B,Hkv,G,d,n,L,s_dim,dtype,tol", FP4_CASES, ids=[c[0] for c in FP4_CASES])
def test_sub_fp4_descriptors_are_the_fp4_storage_of_the_bf16_ones(name, B, Hkv, G, d, n, L, s_dim, dtype, tol):
    """kv_cov_sub4_build writes, bit for bit, what the oracle's FP4 packing makes of the bfloat16
    subspace descriptors (which match the oracle's solve, above), and its scores match the
    oracle's FP4 scores of those bytes."""
    w = W.Workload(name, 4200 + n, B, G * Hkv, Hkv, d, n, L, dtype, 5, "cobs2_sub", True, "clusters", sub_dim=s_dim)
    data = rand_inputs(4200 + n + s_dim, B, G * Hkv, Hkv, d, n, dtype)
    U = basis(w, s_dim)
    q, K, Ud = dev(data["q"]), dev(data["K"]), torch.from_numpy(U).cuda()
    kc = csa.kv_cov_sub_build(K, Ud, L)
    k4 = csa.kv_cov_sub_build(K, Ud, L, fp4=True)
    sc = csa.block_score_cobs2_sub(q, k4, Ud, L, n, fp4=True)
    sel = csa.topk_select(sc, w.k)
    torch.cuda.synchronize()
    shp = oshape(w)
    kc, k4, sc, sel = host(kc), host(k4), host(sc), host(sel)
    assert np.array_equal(k4, O.cov_sub4_pack(shp, kc, s_dim)), f"{name}: FP4 bytes differ"
    ref = O.group_score(shp, O.cobs2_sub4_logits(shp, data["q"], k4, U))
    ref_sel, margin = O.topk_select(ref, w.k)
    err = assert_scores(sc, ref, f"{name} fp4")
    assert_selection(sel, ref_sel, ref, margin, f"{name} fp4", err)


def test_sub_fp4_full_size_all_pairs():
    w = W.WORKLOADS["llama3_8b_layer_b32_cobs2_sub_fp4"]
    data = W.generate(w)
    U = basis(w, w.sub_dim)
    q, K, Ud = dev(data["q"]), dev(data["K"]), torch.from_numpy(U).cuda()
    k4 = csa.kv_cov_sub_build(K, Ud, w.block_size, fp4=True)
    sc = csa.block_score_cobs2_sub(q, k4, Ud, w.block_size, w.n_tokens, fp4=True)
    sel = csa.topk_select(sc, w.k)
    torch.cuda.synchronize()
    shp = oshape(w)
    k4, sc, sel = host(k4), host(sc), host(sel)
    assert k4.shape[-1] == 464
    ref = O.group_score(shp, O.cobs2_sub4_logits(shp, data["q"], k4, U))
    ref_sel, margin = O.topk_select(ref, w.k)
    err = assert_scores(sc, ref, w.name)
    assert_selection(sel, ref_sel, ref, margin, w.name, err)
