"""Parity of the HIP path (through the C-ABI) with the fp64 oracle on the same seeded inputs.

Bars (written here; each follows from fp32 accumulation against the fp64 oracle):
  * summaries and selections: bit-exact;
  * outputs: per row ||o - o_ref||_inf / ||o_ref||_inf <= 2e-3 for bfloat16 inputs, 1e-5 for
    binary32 inputs (fp32 accumulation against fp64);
  * lse: |lse - lse_ref| <= 1e-3 (bfloat16) / 1e-5 (binary32);
  * scores: |s - s_ref| <= 1e-4 + 1e-5 |s_ref| (fp32 dot products and log-sum-exp).
A selection row is near-tied when its oracle margin s_(k) - s_(k+1) is below that same score
bound at s_(k): there the fp32 scores may order the two sides of the boundary either way.  Only
near-tied rows may select differently, and only among blocks whose oracle scores lie within the
bound of s_(k).  Every near-tied row is recorded (parity_report) and printed at the end of the
run, with whether its selection differs.
"""
import numpy as np
import pytest
import torch

import parity_report
from coreset_softmax_attention_amd import csa
from coreset_softmax_attention_amd import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu

OUT_TOL = {"bf16": 2e-3, "f32": 1e-5}
LSE_TOL = {"bf16": 1e-3, "f32": 1e-5}
SCORE_ATOL, SCORE_RTOL = 1e-4, 1e-5


def score_bound(s):
    """The asserted score error at oracle score s."""
    return SCORE_ATOL + SCORE_RTOL * np.abs(s)


def dev(a):
    return csa.to_device(a)


def host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def oshape(w, B=None, Hkv=None):
    B = w.batch if B is None else B
    Hkv = w.n_kv_heads if Hkv is None else Hkv
    return O.Shape(B, Hkv * w.group, Hkv, w.head_dim, w.n_tokens, w.block_size, w.dtype)


def row_err(a, ref):
    a, ref = np.asarray(a, np.float64), np.asarray(ref, np.float64)
    d = a.shape[-1]
    num = np.abs(a - ref).reshape(-1, d).max(axis=1)
    den = np.abs(ref).reshape(-1, d).max(axis=1)
    return float((num / den).max())


def assert_out(out, lse, ref_out, ref_lse, dtype, what=""):
    e = row_err(out, ref_out)
    assert e <= OUT_TOL[dtype], f"{what}: output row error {e:.3e} > {OUT_TOL[dtype]}"
    le = float(np.abs(np.asarray(lse, np.float64) - ref_lse).max())
    assert le <= LSE_TOL[dtype], f"{what}: lse error {le:.3e} > {LSE_TOL[dtype]}"


def assert_scores(s, ref, what=""):
    """Scores within the bound; returns the largest error as a fraction of its bound."""
    s, ref = np.asarray(s, np.float64), np.asarray(ref, np.float64)
    same_inf = np.isinf(s) & (s == ref)  # -inf: a block whose proxy leaves no error
    with np.errstate(invalid="ignore"):
        err = np.where(same_inf, 0.0, np.abs(s - ref))
        bad = ~(err <= score_bound(np.where(same_inf, 0.0, ref)))
    assert not bad.any(), f"{what}: {bad.sum()} scores off, max err {np.nanmax(err):.3e}"
    return float((err / score_bound(np.where(same_inf, 0.0, ref))).max()) if err.size else 0.0


def assert_selection(sel, ref_sel, ref_score, margin, what="", score_err=None):
    """Bit-exact selection except in near-tied rows; records every near-tied row."""
    if ref_sel.shape[-1] == 0:
        assert np.asarray(sel).size == 0, f"{what}: k = 0 selected blocks"
        return
    kk = ref_sel.shape[-1]
    sel = np.asarray(sel).reshape(-1, kk)
    ref_sel = ref_sel.reshape(sel.shape)
    ref_score = np.asarray(ref_score, np.float64).reshape(sel.shape[0], -1)
    margin = np.asarray(margin).reshape(-1)
    kth = -np.sort(-ref_score, axis=1)[:, kk - 1]  # the oracle's k-th largest score per row
    bound = score_bound(kth)
    near = []
    for r in range(sel.shape[0]):
        assert np.all(np.diff(sel[r]) > 0), f"{what}: row {r} not strictly ascending"
        same = np.array_equal(sel[r], ref_sel[r])
        tied = bool(margin[r] < bound[r])
        if tied:
            near.append((r, float(margin[r]), float(bound[r]), not same))
        if same:
            continue
        assert tied, f"{what}: row {r} differs with margin {margin[r]:.3e} >= {bound[r]:.3e}: " \
                     f"{sel[r]} vs {ref_sel[r]}"
        for blk in set(sel[r].tolist()) ^ set(ref_sel[r].tolist()):
            assert abs(ref_score[r, blk] - kth[r]) < bound[r], f"{what}: row {r} block {blk} is not near-tied"
    parity_report.add(what, sel.shape[0], near, score_err)


# ---------------------------------------------------------------------------
# helpers running each side
# ---------------------------------------------------------------------------

def gpu_pipeline(w, data, k=None, mode=None, proxies=None):
    k = w.k if k is None else k
    mode = w.score_mode if mode is None else mode
    proxies = w.proxies if proxies is None else proxies
    q, K, V = dev(data["q"]), dev(data["K"]), dev(data["V"])
    Kbar, Vbar = csa.kv_summary_build(K, V, w.block_size)
    Kbox = csa.kv_box_build(K, w.block_size) if mode == "box" else None
    Kvar = csa.kv_var_build(K, w.block_size) if mode == "proxy_error" else None
    keys = {"summary": Kbar, "exact_mass": K, "box": Kbox, "proxy_error": Kvar}[mode]
    scores = csa.block_score(q, keys, mode, w.block_size, n_tokens=w.n_tokens)
    sel = csa.topk_select(scores, k)
    ti = dev(data["tok_idx"]) if "tok_idx" in data else None
    tw = dev(data["tok_logw"]) if "tok_logw" in data else None
    out, lse = csa.sparse_decode_attn(q, K, V, Kbar, Vbar, sel, w.block_size, proxies=proxies, tok_idx=ti,
                                      tok_logw=tw)
    torch.cuda.synchronize()
    r = {"Kbar": host(Kbar), "Vbar": host(Vbar), "score": host(scores), "sel": host(sel), "out": host(out),
         "lse": host(lse)}
    if Kbox is not None:
        r["Kbox"] = host(Kbox)
    if Kvar is not None:
        r["Kvar"] = host(Kvar)
    return r


def oracle_pipeline(w, data, k=None, mode=None, proxies=None):
    k = w.k if k is None else k
    mode = w.score_mode if mode is None else mode
    proxies = w.proxies if proxies is None else proxies
    B = data["q"].shape[0]
    shp = oshape(w, B=B, Hkv=data["K"].shape[1])
    Kbar, Vbar = O.kv_summary_build(shp, data["K"], data["V"])
    Kbox = O.kv_box_build(shp, data["K"]) if mode == "box" else None
    Kvar = O.var_build(shp, data["K"], Kbar) if mode == "proxy_error" else None
    md = {"summary": O.SUMMARY, "exact_mass": O.EXACT_MASS, "box": O.BOX, "proxy_error": O.PROXY_ERROR}[mode]
    keys = {"summary": Kbar, "exact_mass": data["K"], "box": Kbox, "proxy_error": Kvar}[mode]
    score = O.block_score(shp, md, data["q"], keys)
    sel, margin = O.topk_select(score, k)
    out, lse = O.sparse_decode_attn(shp, data["q"], data["K"], data["V"], Kbar, Vbar, sel, proxies,
                                    data.get("tok_idx"), data.get("tok_logw"))
    r = {"Kbar": Kbar, "Vbar": Vbar, "score": score, "sel": sel, "margin": margin, "out": out, "lse": lse}
    if Kbox is not None:
        r["Kbox"] = Kbox
    if Kvar is not None:
        r["Kvar"] = Kvar
    return r


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def compare_pipelines(w, g, o, what):
    assert np.array_equal(bits(g["Kbar"]), bits(o["Kbar"])), f"{what}: Kbar not bit-exact"
    assert np.array_equal(bits(g["Vbar"]), bits(o["Vbar"])), f"{what}: Vbar not bit-exact"
    if "Kbox" in o:
        assert np.array_equal(bits(g["Kbox"]), bits(o["Kbox"])), f"{what}: Kbox not bit-exact"
    if "Kvar" in o:
        assert np.array_equal(bits(g["Kvar"]), bits(o["Kvar"])), f"{what}: Kvar not bit-exact"
    err = assert_scores(g["score"], o["score"], what)
    assert_selection(g["sel"], o["sel"], o["score"], o["margin"], what, err)
    assert_out(g["out"], g["lse"], o["out"], o["lse"], w.dtype, what)


def rand_inputs(seed, B, Hq, Hkv, d, n, dtype, qscale=2.0):
    rng = np.random.default_rng(seed)

    def st(x):
        return x.astype(np.float32) if dtype == "f32" else W.to_bf16_bits(x.astype(np.float32))

    return {"q": st(qscale * rng.standard_normal((B, Hq, d))), "K": st(rng.standard_normal((B, Hkv, n, d))),
            "V": st(rng.standard_normal((B, Hkv, n, d)))}


def small(name, **kw):
    return W.scaled_down(W.WORKLOADS[name], **kw)


# ---------------------------------------------------------------------------
# small cases: several tiles, ragged tails, every mode
# ---------------------------------------------------------------------------

SMALL = [
    ("tiny_f32_d64", W.WORKLOADS["tiny_f32_d64"]),
    ("llama_b2_4k", small("llama3_8b_layer_b1", batch=2, n_tokens=4096, n_kv_heads=2)),
    ("mha_exact_4k", small("exact_mass_mha_b8", batch=2, n_tokens=4096, n_kv_heads=3)),
    ("gqa_exact_4k", small("exact_mass_gqa_b8", batch=2, n_tokens=4096, n_kv_heads=2)),
    ("coreset_g7_8k", small("weighted_coreset_128k", batch=2, n_tokens=8192, n_kv_heads=2).with_(coreset=300)),
    ("box_b2_4k", small("llama3_8b_layer_b32_box", batch=2, n_tokens=4096, n_kv_heads=2)),
]


@pytest.mark.parametrize("name,w", SMALL, ids=[s[0] for s in SMALL])
def test_pipeline_small(name, w):
    data = W.generate(w)
    compare_pipelines(w, gpu_pipeline(w, data), oracle_pipeline(w, data), name)


@pytest.mark.parametrize("mode", ["summary", "exact_mass", "box"])
@pytest.mark.parametrize("proxies", [True, False])
def test_tiny_mode_matrix(mode, proxies):
    """Single-head fp32 decode: {summary, exact mass} x {proxies, discard} at k = 8, and keeping
    all 64 blocks, which must equal dense attention."""
    w = W.WORKLOADS["tiny_f32_d64"]
    data = W.generate(w)
    compare_pipelines(w, gpu_pipeline(w, data, mode=mode, proxies=proxies),
                      oracle_pipeline(w, data, mode=mode, proxies=proxies), f"tiny {mode} {proxies}")
    g_all = gpu_pipeline(w, data, k=w.n_blocks, mode=mode, proxies=proxies)
    ref, ref_lse = O.dense_decode_attn(oshape(w), data["q"], data["K"], data["V"])
    assert_out(g_all["out"], g_all["lse"], ref, ref_lse, "f32", "all blocks vs dense")


@pytest.mark.parametrize("dtype,G,d,n,L", [
    ("bf16", 3, 128, 1000, 64),    # ragged last block (40 tokens), odd group
    ("f32", 2, 64, 777, 16),       # ragged (9 tokens), fp32, d = 64
    ("bf16", 1, 64, 2048, 32),     # MHA, d = 64
    ("bf16", 12, 128, 1536, 64),   # group of 12: two head chunks (8 + 4)
    ("bf16", 4, 128, 100, 256),    # one block longer than the cache
    ("f32", 2, 128, 300, 1),       # blocks of one token: proxies exact
])
def test_pipeline_shapes(dtype, G, d, n, L):
    Hkv = 2
    w = W.Workload("shape_case", 0, 2, G * Hkv, Hkv, d, n, L, dtype, 3, "summary", True, "clusters")
    data = rand_inputs(100 + G + d + n, 2, G * Hkv, Hkv, d, n, dtype)
    for mode in ("summary", "exact_mass", "box"):
        for proxies in (True, False):
            k = min(3, w.n_blocks)
            compare_pipelines(w.with_(k=k), gpu_pipeline(w, data, k=k, mode=mode, proxies=proxies),
                              oracle_pipeline(w, data, k=k, mode=mode, proxies=proxies),
                              f"{dtype} G={G} d={d} n={n} L={L} {mode} {proxies}")


@pytest.mark.parametrize("k", [0, 1, 7, 16])
def test_sparse_edge_k(k):
    """k = 0 (proxies only), a single block, and every block (proxies all masked)."""
    w = W.Workload("edge_k", 0, 2, 8, 2, 128, 1024, 64, "bf16", k, "summary", True, "clusters")
    data = rand_inputs(7 + k, 2, 8, 2, 128, 1024, "bf16")
    compare_pipelines(w, gpu_pipeline(w, data), oracle_pipeline(w, data), f"k={k}")
    if k == 16:
        ref, ref_lse = O.dense_decode_attn(oshape(w), data["q"], data["K"], data["V"])
        g = gpu_pipeline(w, data)
        assert_out(g["out"], g["lse"], ref, ref_lse, "bf16", "all blocks + masked proxies vs dense")


def topk_by_rule(scores, k):
    """The k largest scores per row, ties to the lower index, ascending (the selection rule)."""
    s2 = scores.reshape(-1, scores.shape[-1])
    out = np.empty((s2.shape[0], k), np.int32)
    for r, row in enumerate(s2):
        order = np.lexsort((np.arange(row.size), -row.astype(np.float64)))
        out[r] = np.sort(order[:k])
    return out.reshape(scores.shape[:-1] + (k,))


@pytest.mark.parametrize("n,k", [(65536, 8), (131072, 32), (40000, 5)])
def test_selection_ties_across_waves(n, k):
    """Equal block scores far apart: the cache repeats every 256 blocks, so each score occurs
    several times, in the shares of different waves of the two-level top-k.  The selection
    must follow the rule on the GPU's own scores exactly: the k largest, ties to the lower
    index (few KV heads: the split score kernels and the group-score kernel select)."""
    B, Hkv, G, d, L = 1, 2, 4, 128, 64
    rng = np.random.default_rng(n + k)
    period = 256 * L
    base = rng.standard_normal((B, Hkv, period, d)).astype(np.float32)
    K = np.concatenate([base] * (-(-n // period)), axis=2)[:, :, :n]
    data = {"q": W.to_bf16_bits(2.0 * rng.standard_normal((B, G * Hkv, d)).astype(np.float32)),
            "K": W.to_bf16_bits(K), "V": W.to_bf16_bits(rng.standard_normal((B, Hkv, n, d)).astype(np.float32))}
    q, Kd, Vd = dev(data["q"]), dev(data["K"]), dev(data["V"])
    Kbar, Vbar = csa.kv_summary_build(Kd, Vd, L)
    _, _, sc, sel = csa.selective_decode_step(q, Kd, Vd, Kbar, Vbar, k, L, want_scores=True, want_sel=True)
    sc2 = csa.block_score(q, Kbar, "summary", L, n_tokens=n)
    sel2 = csa.topk_select(sc2, k)
    torch.cuda.synchronize()
    sc, sel, sc2, sel2 = host(sc), host(sel), host(sc2), host(sel2)
    assert np.array_equal(bits(sc), bits(sc2))
    nb = sc.shape[-1]
    full = nb // 256 * 256
    assert (sc[..., :full].reshape(B, Hkv, -1, 256) == sc[..., None, :256]).all(), "repeated blocks score alike"
    want = topk_by_rule(sc, k)
    assert np.array_equal(sel, want), f"step selection {sel} != rule {want}"
    assert np.array_equal(sel2, want), f"topk_select {sel2} != rule {want}"


def test_weighted_tokens_only_and_duplicates():
    """A weighted token list alone (k = 0, no proxies), with repeated indices."""
    B, Hkv, G, d, n, L, m = 2, 2, 4, 128, 2048, 64, 700
    data = rand_inputs(31, B, G * Hkv, Hkv, d, n, "bf16")
    rng = np.random.default_rng(32)
    idx = rng.integers(0, n, (B, Hkv, m)).astype(np.int32)
    lw = rng.standard_normal((B, Hkv, m)).astype(np.float32)
    shp = O.Shape(B, G * Hkv, Hkv, d, n, L, "bf16")
    sel = np.zeros((B, Hkv, 0), np.int32)
    ref, ref_lse = O.sparse_decode_attn(shp, data["q"], data["K"], data["V"], None, None, sel, False, idx, lw)
    out, lse = csa.sparse_decode_attn(dev(data["q"]), dev(data["K"]), dev(data["V"]), None, None, None, L,
                                      proxies=False, tok_idx=dev(idx), tok_logw=dev(lw))
    assert_out(host(out), host(lse), ref, ref_lse, "bf16", "weighted only")


@pytest.mark.parametrize("dtype,G,n", [("bf16", 4, 5000), ("f32", 1, 3000), ("bf16", 7, 4096)])
def test_dense_matches_oracle(dtype, G, n):
    B, Hkv, d = 2, 2, 128
    data = rand_inputs(40 + G, B, G * Hkv, Hkv, d, n, dtype)
    ref, ref_lse = O.dense_decode_attn(O.Shape(B, G * Hkv, Hkv, d, n, 64, dtype), data["q"], data["K"], data["V"])
    out, lse = csa.dense_decode_attn(dev(data["q"]), dev(data["K"]), dev(data["V"]))
    assert_out(host(out), host(lse), ref, ref_lse, dtype, "dense")


def test_keeping_all_blocks_equals_gpu_dense():
    w = small("llama3_8b_layer_b1", batch=2, n_tokens=4096, n_kv_heads=2)
    data = W.generate(w)
    g = gpu_pipeline(w, data, k=w.n_blocks, proxies=False)
    out, lse = csa.dense_decode_attn(dev(data["q"]), dev(data["K"]), dev(data["V"]))
    assert_out(g["out"], g["lse"], host(out).astype(np.float64), host(lse).astype(np.float64), "bf16",
               "all blocks vs GPU dense")


def test_equal_logit_tail_is_exact_on_gpu():
    """The page's exactness case, through the kernels: q is zero on half its coordinates and the
    tail keys agree on the other half, so every proxy carries its block's mass exactly."""
    d, n, L = 64, 256, 16
    rng = np.random.default_rng(10)
    q = np.zeros((1, 1, d))
    q[0, 0, : d // 2] = rng.integers(-8, 9, d // 2) / 4
    K = rng.integers(-8, 9, (1, 1, n, d)) / 4
    V = rng.integers(-8, 9, (1, 1, n, d)) / 4
    k0 = rng.integers(-8, 9, d // 2) / 4
    for b in range(n // L):
        if b not in (2, 7):
            K[0, 0, b * L:(b + 1) * L, : d // 2] = k0
    q, K, V = (x.astype(np.float32) for x in (q, K, V))
    Kb, Vb = csa.kv_summary_build(dev(K), dev(V), L)
    sel = dev(np.array([[[2, 7]]], np.int32))
    out, lse = csa.sparse_decode_attn(dev(q), dev(K), dev(V), Kb, Vb, sel, L, proxies=True)
    ref, ref_lse = O.dense_decode_attn(O.Shape(1, 1, 1, d, n, L, "f32"), q, K, V)
    assert_out(host(out), host(lse), ref, ref_lse, "f32", "equal-logit tail")


def test_topk_ties_and_sizes():
    """Generated fp32 score rows with planted ties (including +0 / -0) against the oracle's
    top-k on the same values: bit-exact."""
    rng = np.random.default_rng(50)
    for nb in (1, 5, 9, 64, 100, 512, 513, 1000, 2048, 4099):
        s = rng.standard_normal((6, nb)).astype(np.float32)
        s[1] = np.round(s[1] * 2) / 2  # many exact ties
        s[2] = 0.0
        s[2, ::3] = -0.0
        s[3] = np.float32(1.5)
        s[4, : nb // 2] = np.float32(-3.0)
        s[5] = np.arange(nb, dtype=np.float32)  # the largest scores all in the last blocks
        t = torch.from_numpy(s).cuda()
        for k in sorted({0, 1, 2, 3, 5, 8, 9, 16, nb // 2, nb - 1, nb, nb + 3}):
            if k < 0:
                continue
            got = host(csa.topk_select(t, k))
            ref, _ = O.topk_select(s.astype(np.float64), k)
            assert np.array_equal(got, ref), (nb, k)


def test_runs_are_bitwise_reproducible():
    w = small("llama3_8b_layer_b1", batch=2, n_tokens=8192, n_kv_heads=2)
    data = W.generate(w)
    a, b = gpu_pipeline(w, data), gpu_pipeline(w, data)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_index_checks_reject_what_the_oracle_rejects():
    """With csa_set_index_checks on, selections that name a block twice or outside [0, nb), and
    weighted tokens outside [0, n), are rejected on the host before any launch, as the oracle
    rejects them; valid lists give the same bits as without the checks."""
    B, Hkv, G, d, n, L = 2, 2, 4, 128, 1024, 64
    nb = n // L
    data = rand_inputs(901, B, G * Hkv, Hkv, d, n, "bf16")
    shp = O.Shape(B, G * Hkv, Hkv, d, n, L, "bf16")
    q, K, V = dev(data["q"]), dev(data["K"]), dev(data["V"])
    Kbar, Vbar = csa.kv_summary_build(K, V, L)
    Kb_o, Vb_o = O.kv_summary_build(shp, data["K"], data["V"])
    good = np.tile(np.array([1, 4, 9], np.int32), (B, Hkv, 1))
    tok = np.tile(np.array([3, 500, 1023], np.int32), (B, Hkv, 1))
    logw = np.zeros((B, Hkv, 3), np.float32)
    bad_sels = [good.copy(), good.copy(), good.copy()]
    bad_sels[0][1, 0] = [4, 4, 9]       # a block twice
    bad_sels[1][0, 1, 2] = nb          # past the last block
    bad_sels[2][1, 1, 0] = -1          # negative
    bad_tok = tok.copy()
    bad_tok[1, 0, 1] = n
    prev = csa.set_index_checks(True)
    try:
        for sel in bad_sels:
            with pytest.raises(ValueError):
                O.sparse_decode_attn(shp, data["q"], data["K"], data["V"], Kb_o, Vb_o, sel, True)
            with pytest.raises(csa.CsaError, match="sel") as e:
                csa.sparse_decode_attn(q, K, V, Kbar, Vbar, dev(sel), L, proxies=True)
            assert e.value.status == csa.CSA_ERR_INVALID_ARG
        with pytest.raises(ValueError):
            O.sparse_decode_attn(shp, data["q"], data["K"], data["V"], Kb_o, Vb_o, good, True, bad_tok, logw)
        with pytest.raises(csa.CsaError, match="tok_idx") as e:
            csa.sparse_decode_attn(q, K, V, Kbar, Vbar, dev(good), L, proxies=True, tok_idx=dev(bad_tok),
                                   tok_logw=dev(logw))
        assert e.value.status == csa.CSA_ERR_INVALID_ARG
        with pytest.raises(csa.CsaError, match="tok_idx"):
            csa.selective_decode_step(q, K, V, Kbar, Vbar, 3, L, tok_idx=dev(bad_tok), tok_logw=dev(logw))
        checked = csa.sparse_decode_attn(q, K, V, Kbar, Vbar, dev(good), L, proxies=True, tok_idx=dev(tok),
                                         tok_logw=dev(logw))
        torch.cuda.synchronize()
    finally:
        csa.set_index_checks(prev)
    plain = csa.sparse_decode_attn(q, K, V, Kbar, Vbar, dev(good), L, proxies=True, tok_idx=dev(tok),
                                   tok_logw=dev(logw))
    torch.cuda.synchronize()
    for a, b in zip(checked, plain):
        assert np.array_equal(bits(host(a)), bits(host(b)))


def test_invalid_arguments_raise():
    q = torch.zeros((1, 4, 96), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros((1, 2, 64, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(csa.CsaError, match="head_dim 96"):
        csa.dense_decode_attn(q, K, K)


# ---------------------------------------------------------------------------
# the full-size workloads, in the launch configuration the benchmark times;
# the oracle recomputes every (b, KV head) pair
# ---------------------------------------------------------------------------

FULL = ["llama3_8b_layer_b1", "llama3_8b_layer_b32", "exact_mass_mha_b8", "exact_mass_gqa_b8",
        "weighted_coreset_128k", "llama3_8b_layer_b32_box", "llama3_8b_layer_b32_err", "g8_layer_b32"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_all_pairs(name):
    """Every (b, KV head) pair of the full-size workload: summaries (and box or variance
    tokens) bit for bit, scores within the bound, selections bit for bit outside near-tied
    rows, outputs per row; through the three entry points and, for the summary and
    exact-mass scores, through selective_decode_step as the benchmark calls it."""
    w = W.WORKLOADS[name]
    data = W.generate(w)
    o = oracle_pipeline(w, data)
    g = gpu_pipeline(w, data)
    assert np.isfinite(g["out"]).all() and np.isfinite(g["lse"]).all()
    compare_pipelines(w, g, o, f"{name} (three entry points)")
    if w.score_mode in ("summary", "exact_mass"):
        st = gpu_step(w, data)
        compare_pipelines(w, st, o, f"{name} (selective_decode_step)")
        assert np.array_equal(st["sel"], g["sel"]), f"{name}: the step and the three calls select differently"


def test_graph_replay_matches_eager():
    """The decode step captured in a HIP graph and replayed several times, with eager work on
    the same buffers between replays, reproduces the eager result bit for bit each time."""
    w = small("llama3_8b_layer_b1", batch=4, n_tokens=8192, n_kv_heads=2)
    data = W.generate(w)
    q, K, V = dev(data["q"]), dev(data["K"]), dev(data["V"])
    Kbar, Vbar = csa.kv_summary_build(K, V, w.block_size)
    shape = csa.make_shape(q, K, w.block_size)
    scores = torch.empty((w.batch, w.n_kv_heads, w.n_blocks), dtype=torch.float32, device="cuda")
    sel = torch.empty((w.batch, w.n_kv_heads, w.k), dtype=torch.int32, device="cuda")
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.batch, w.n_q_heads), dtype=torch.float32, device="cuda")
    ws_s = torch.empty(max(1, csa.workspace_size(shape, csa.CSA_WS_BLOCK_SCORE_SUMMARY)), dtype=torch.uint8,
                       device="cuda")
    ws_a = torch.empty(max(1, csa.workspace_size(shape, csa.CSA_WS_SPARSE_DECODE_ATTN, w.k, 0)),
                       dtype=torch.uint8, device="cuda")

    def step():
        csa.block_score(q, Kbar, "summary", w.block_size, n_tokens=w.n_tokens, scores=scores, ws=ws_s)
        csa.topk_select(scores, w.k, sel=sel)
        csa.sparse_decode_attn(q, K, V, Kbar, Vbar, sel, w.block_size, out=out, lse=lse, ws=ws_a)

    step()
    torch.cuda.synchronize()
    ref = [host(t).copy() for t in (scores, sel, out, lse)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        for t in (scores, out, lse):
            t.fill_(float(i))
        sel.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (scores, sel, out, lse)):
            assert np.array_equal(bits(a), bits(host(b))), f"replay {i}"


# ---------------------------------------------------------------------------
# the one-call decode step (one kernel per KV head where the shape allows)
# ---------------------------------------------------------------------------

def gpu_step(w, data, k=None, mode=None, proxies=None):
    k = w.k if k is None else k
    mode = w.score_mode if mode is None else mode
    proxies = w.proxies if proxies is None else proxies
    q, K, V = dev(data["q"]), dev(data["K"]), dev(data["V"])
    Kbar, Vbar = csa.kv_summary_build(K, V, w.block_size)
    ti = dev(data["tok_idx"]) if "tok_idx" in data else None
    tw = dev(data["tok_logw"]) if "tok_logw" in data else None
    out, lse, scores, sel = csa.selective_decode_step(q, K, V, Kbar, Vbar, k, w.block_size, mode=mode,
                                                      proxies=proxies, tok_idx=ti, tok_logw=tw, want_scores=True,
                                                      want_sel=True)
    torch.cuda.synchronize()
    return {"Kbar": host(Kbar), "Vbar": host(Vbar), "score": host(scores), "sel": host(sel), "out": host(out),
            "lse": host(lse)}


# B * Hkv >= 32 takes the one-kernel path, and so does a small share per KV head
# ((proxies + k L + m) G <= 4096); the rest runs the split kernels
STEP_CASES = [
    ("llama_b8_4k", small("llama3_8b_layer_b32", batch=8, n_tokens=4096, n_kv_heads=4), {}),
    ("llama_b8_4k_k32", small("llama3_8b_layer_b32", batch=8, n_tokens=4096, n_kv_heads=4), {"k": 32}),
    ("llama_b8_4k_k0", small("llama3_8b_layer_b32", batch=8, n_tokens=4096, n_kv_heads=4), {"k": 0}),
    ("llama_b8_discard", small("llama3_8b_layer_b32", batch=8, n_tokens=4096, n_kv_heads=4), {"proxies": False}),
    ("mha_b8_summary", small("exact_mass_mha_b8", batch=2, n_tokens=4096, n_kv_heads=16),
     {"mode": "summary", "proxies": True}),
    ("coreset_g7_b8", small("weighted_coreset_128k", batch=8, n_tokens=8192, n_kv_heads=4).with_(coreset=300), {}),
    # 640 blocks of 16: 20 proxy tiles (three for waves 0-3, two for the others) and 6 exact
    # tiles, so odd and even tile counts, and waves without exact tiles, meet in one launch
    ("llama_b8_L16_nb640", small("llama3_8b_layer_b32", batch=8, n_tokens=10240, n_kv_heads=4).with_(block_size=16),
     {"k": 12}),
    # 1024 blocks: more than 16 mean-key tiles, so waves take more than two proxy tiles each
    ("llama_b8_8k_L8", small("llama3_8b_layer_b32", batch=8, n_tokens=8192, n_kv_heads=4).with_(block_size=8),
     {"k": 24}),
    # G = 8 heads over 512 blocks: the largest logit table in LDS
    ("g8_d64_nb512", W.Workload("g8_d64_nb512", 1003, 4, 64, 8, 64, 8192, 16, "bf16", 12, "summary", True,
                                "clusters"), {}),
    # four KV heads: (59 + 320) x 4 rows x heads, one kernel; with k = 16, (48 + 1024) x 4 > 4096, split
    ("few_pairs_small_share", small("llama3_8b_layer_b1", batch=2, n_tokens=4096, n_kv_heads=2), {}),
    ("few_pairs_unfused", small("llama3_8b_layer_b1", batch=2, n_tokens=4096, n_kv_heads=2), {"k": 16}),
    ("exact_mass_unfused", small("exact_mass_gqa_b8", batch=8, n_tokens=4096, n_kv_heads=4), {}),
]


@pytest.mark.parametrize("name,w,kw", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_decode_step_matches_oracle(name, w, kw):
    data = W.generate(w)
    compare_pipelines(w.with_(**{k: v for k, v in kw.items() if k == "k"}), gpu_step(w, data, **kw),
                      oracle_pipeline(w, data, **kw), name)


def large_nb_inputs(seed, nb, keys):
    """One sequence, 2 KV heads of 8 query heads, d = 64, blocks of 64.  keys: "random";
    "ties" (blocks 300, 700 and 1000 mod nb hold the same keys, pointed along their group's
    mean query: they tie for the top score); "equal" (all keys zero: every block ties)."""
    B, Hq, Hkv, d, L = 1, 16, 2, 64, 64
    n = nb * L
    data = rand_inputs(seed, B, Hq, Hkv, d, n, "bf16")
    if keys == "random":
        return data
    rng = np.random.default_rng(seed + 1)
    if keys == "equal":
        K = np.zeros((B, Hkv, n, d), np.float32)
    else:
        q = (data["q"].astype(np.uint32) << 16).view(np.float32).reshape(B, Hkv, Hq // Hkv, d)
        K = 0.1 * rng.standard_normal((B, Hkv, n, d)).astype(np.float32)
        top = 3.0 * q.mean(axis=2)[:, :, None, :] + 0.1 * rng.standard_normal((B, Hkv, L, d))
        for blk in sorted({700 % nb, 300 % nb, 1000 % nb}):
            K[:, :, blk * L:(blk + 1) * L] = top
    data["K"] = W.to_bf16_bits(K)
    return data


@pytest.mark.parametrize("keys", ["random", "ties", "equal"])
@pytest.mark.parametrize("nb,k", [(600, 1), (600, 8), (1024, 3), (2048, 5), (2048, 8), (2048, 9)])
def test_split_step_selection_beyond_512_blocks(nb, k, keys):
    """selective_decode_step on the split kernels (2 KV heads of 8 query heads) with more than
    512 blocks, where the group-score kernel ranks with one wave over up to 32 scores per lane:
    candidates from the bound of the lane maxima, or rounds of wave-wide maxima when that bound
    admits more than 64 (every block tied).  Against the oracle, and scores and selection bit for
    bit against block_score + topk_select."""
    w = W.Workload("large_nb", 0, 1, 16, 2, 64, nb * 64, 64, "bf16", k, "summary", True, "clusters")
    data = large_nb_inputs(500 + nb + k, nb, keys)
    g, m = gpu_step(w, data), gpu_pipeline(w, data)
    assert np.array_equal(bits(g["score"]), bits(m["score"])), "scores differ from block_score"
    assert np.array_equal(g["sel"], m["sel"]), "selection differs from topk_select"
    if keys == "equal":
        assert (g["sel"] == np.arange(k)).all()
    if keys == "ties" and k == 1:
        assert (g["sel"] == min(700 % nb, 300 % nb, 1000 % nb)).all()
    compare_pipelines(w, g, oracle_pipeline(w, data), f"split step nb={nb} k={k} {keys}")


# The same route at other shapes: one query head per KV head over a ragged last chunk of
# candidates, the weighted-coreset recipe scaled down (G = 7, weighted tokens, k = 32: a
# chunk's whole candidate list), and no proxies (only exact rows: every first tile waits for
# the ranking)
RANKED_CASES = [
    ("g1_nb700", W.Workload("ranked_g1", 0, 2, 3, 3, 128, 700 * 16, 16, "bf16", 4, "summary", True, "clusters"), {}),
    ("coreset_g7_nb1500_k32",
     small("weighted_coreset_128k", batch=2, n_tokens=1500 * 64, n_kv_heads=2).with_(coreset=300, k=32), {}),
    ("g4_nb2048_no_proxies", W.Workload("ranked_g4", 0, 1, 8, 2, 128, 2048 * 32, 32, "bf16", 6, "summary", False,
                                        "clusters"), {}),
    # six heads over 1001 blocks (not a multiple of 4): the proxy rows read their mean keys
    ("g6_nb1001", W.Workload("ranked_g6", 0, 1, 12, 2, 64, 1001 * 64, 64, "bf16", 5, "summary", True, "clusters"), {}),
]


@pytest.mark.parametrize("name,w,kw", RANKED_CASES, ids=[c[0] for c in RANKED_CASES])
def test_split_step_ranked_shapes(name, w, kw):
    """More than 512 blocks and fewer than 32 KV heads: chunk candidates ranked by the attention
    kernel.  Scores and selection bit for bit against block_score + topk_select, and against the
    oracle."""
    data = W.generate(w)
    g, m = gpu_step(w, data, **kw), gpu_pipeline(w, data, **kw)
    assert np.array_equal(bits(g["score"]), bits(m["score"])), f"{name}: scores differ from block_score"
    assert np.array_equal(g["sel"], m["sel"]), f"{name}: selection differs from topk_select"
    compare_pipelines(w, g, oracle_pipeline(w, data, **kw), name)


@pytest.mark.parametrize("dtype,G,d,n,L", [("bf16", 3, 128, 1000, 64), ("bf16", 8, 64, 2000, 32),
                                           ("bf16", 1, 128, 700, 16)])
def test_decode_step_shapes(dtype, G, d, n, L):
    """Ragged last blocks, d = 64, G = 8 and G = 1 through the one-kernel path."""
    B, Hkv = 8, 4
    w = W.Workload("step_shape", 0, B, G * Hkv, Hkv, d, n, L, dtype, 4, "summary", True, "clusters")
    data = rand_inputs(300 + G + n, B, G * Hkv, Hkv, d, n, dtype)
    compare_pipelines(w, gpu_step(w, data), oracle_pipeline(w, data), f"step G={G} d={d} n={n} L={L}")


def test_decode_step_scores_and_selection_equal_modular_path():
    """The one-kernel step ranks with exactly the scores block_score computes and selects what
    topk_select selects (bit for bit); outputs agree with sparse_decode_attn to rounding."""
    w = small("llama3_8b_layer_b32", batch=8, n_tokens=8192, n_kv_heads=4)
    data = W.generate(w)
    a, b = gpu_step(w, data), gpu_pipeline(w, data)
    assert np.array_equal(bits(a["score"]), bits(b["score"]))
    assert np.array_equal(a["sel"], b["sel"])
    assert row_err(a["out"], b["out"]) < 1e-5
    assert np.abs(a["lse"] - b["lse"]).max() < 1e-5


# ---------------------------------------------------------------------------
# second-order (COBS) descriptors and scores
# ---------------------------------------------------------------------------

def check_cov_descriptors(kc, K, shp, what, tol):
    """Row 0 is the oracle's mean key bit for bit; rows 1.. span the same top eigenspace as the
    oracle's fp64 eigen-solve: sum_i xi_i xi_i^T agrees within `tol` (relative Frobenius) on every
    block whose 4th and 5th eigenvalues are apart (elsewhere the top-4 space is not unique)."""
    Kbar_o, _ = O.kv_summary_build(shp, K, K)
    assert np.array_equal(bits(kc[:, :, :, 0]), bits(Kbar_o)), f"{what}: mean rows not bit-exact"
    ko = O.cov_build(shp, K, Kbar_o)
    Kf = O.widen(shp, K)
    L, n, r = shp.block_size, shp.n_tokens, O.COBS_RANK
    checked = 0
    for b in range(kc.shape[0]):
        for j in range(kc.shape[1]):
            for blk in range(shp.n_blocks):
                X = Kf[b, j, blk * L:min(n, (blk + 1) * L)]
                lam = np.linalg.eigvalsh(np.cov(X.T, bias=True))[::-1] if X.shape[0] > 1 else np.zeros(r + 1)
                if lam[0] > 0 and lam[r - 1] > 1e-5 * lam[0] and (lam[r - 1] - lam[r]) < 1e-2 * lam[0]:
                    continue  # a 4th direction that is both weighty and not unique
                A, B = O.widen(shp, kc[b, j, blk, 1:]), O.widen(shp, ko[b, j, blk, 1:])
                PA, PB = A.T @ A, B.T @ B
                ref = max(np.linalg.norm(PB), 1e-30)
                assert np.linalg.norm(PA - PB) <= tol * ref, f"{what}: block ({b},{j},{blk}) eigenspace differs"
                checked += 1
    assert checked >= 0.8 * kc.shape[0] * kc.shape[1] * shp.n_blocks, f"{what}: too few blocks checked"


COV_CASES = [
    ("f32_d64_L16", W.Workload("c", 0, 1, 2, 2, 64, 700, 16, "f32", 3, "cobs2", True, "clusters"), 1e-4),
    ("bf16_d128_L64", small("llama3_8b_layer_b32", batch=2, n_tokens=4096, n_kv_heads=2), 2e-2),
    ("bf16_d128_ragged", W.Workload("c", 0, 2, 4, 2, 128, 1000, 64, "bf16", 3, "cobs2", True, "clusters"), 2e-2),
    ("bf16_d64_L4", W.Workload("c", 0, 1, 2, 1, 64, 256, 4, "bf16", 3, "cobs2", True, "clusters"), 2e-2),
]


@pytest.mark.parametrize("name,w,tol", COV_CASES, ids=[c[0] for c in COV_CASES])
def test_cov_descriptors_match_oracle(name, w, tol):
    data = W.generate(w) if w.name != "c" else rand_inputs(200 + w.n_tokens, w.batch, w.n_q_heads, w.n_kv_heads,
                                                            w.head_dim, w.n_tokens, w.dtype)
    kc = host(csa.kv_cov_build(dev(data["K"]), w.block_size))
    torch.cuda.synchronize()
    check_cov_descriptors(kc, data["K"], oshape(w, B=data["K"].shape[0], Hkv=data["K"].shape[1]), name, tol)


def cobs2_case(w, data, k=None, proxies=True):
    """GPU pipeline with second-order scores; the oracle scores the GPU's stored descriptors."""
    k = w.k if k is None else k
    q, K, V = dev(data["q"]), dev(data["K"]), dev(data["V"])
    Kbar, Vbar = csa.kv_summary_build(K, V, w.block_size)
    Kcov = csa.kv_cov_build(K, w.block_size)
    scores = csa.block_score(q, Kcov, "cobs2", w.block_size, n_tokens=w.n_tokens)
    sel = csa.topk_select(scores, k)
    out, lse = csa.sparse_decode_attn(q, K, V, Kbar, Vbar, sel, w.block_size, proxies=proxies)
    torch.cuda.synchronize()
    g = {"Kbar": host(Kbar), "Vbar": host(Vbar), "score": host(scores), "sel": host(sel), "out": host(out),
         "lse": host(lse), "Kcov": host(Kcov)}
    shp = oshape(w, B=data["q"].shape[0], Hkv=data["K"].shape[1])
    Kbar_o, Vbar_o = O.kv_summary_build(shp, data["K"], data["V"])
    score = O.group_score(shp, O.cobs2_logits(shp, data["q"], g["Kcov"]))
    sel_o, margin = O.topk_select(score, k)
    out_o, lse_o = O.sparse_decode_attn(shp, data["q"], data["K"], data["V"], Kbar_o, Vbar_o, sel_o, proxies)
    o = {"Kbar": Kbar_o, "Vbar": Vbar_o, "score": score, "sel": sel_o, "margin": margin, "out": out_o, "lse": lse_o}
    return g, o


@pytest.mark.parametrize("B,Hkv,G,n,L,k", [
    (2, 2, 4, 4096, 64, 5),     # split scoring path (few KV heads)
    (8, 4, 4, 4096, 64, 5),     # one workgroup per KV head
    (2, 2, 7, 3000, 64, 8),     # G = 7, ragged last block
    (2, 2, 1, 2048, 32, 3),     # one head per KV head, d = 128
])
def test_cobs2_pipeline_matches_oracle(B, Hkv, G, n, L, k):
    w = W.Workload("cobs2_case", 0, B, G * Hkv, Hkv, 128, n, L, "bf16", k, "cobs2", True, "clusters")
    data = rand_inputs(300 + B + G + n, B, G * Hkv, Hkv, 128, n, "bf16")
    g, o = cobs2_case(w, data)
    compare_pipelines(w, g, o, f"cobs2 B={B} Hkv={Hkv} G={G} n={n} L={L}")


@pytest.mark.parametrize("B,Hkv,G,n,L,k", [
    (2, 2, 4, 2048, 32, 4),     # d = 64, split scoring path
    (2, 1, 1, 1000, 16, 3),     # d = 64, one head per KV head, ragged
])
def test_cobs2_pipeline_d64_matches_oracle(B, Hkv, G, n, L, k):
    """The second-order split kernel at d = 64 (eight lanes per descriptor row in its loads)."""
    w = W.Workload("cobs2_d64", 0, B, G * Hkv, Hkv, 64, n, L, "bf16", k, "cobs2", True, "clusters")
    data = rand_inputs(310 + B + G + n, B, G * Hkv, Hkv, 64, n, "bf16")
    g, o = cobs2_case(w, data)
    compare_pipelines(w, g, o, f"cobs2 d=64 B={B} Hkv={Hkv} G={G} n={n} L={L}")


def test_cov4_descriptors_are_the_fp4_storage_of_the_bf16_ones():
    """kv_cov4_build stores exactly what the oracle's FP4 packing makes of kv_cov_build's
    bfloat16 descriptors (same eigen-solve on the GPU): bit for bit, d = 128 and 64, ragged."""
    # L = 3: at most two nonzero eigenvectors, the others have scale 0 and zero codes
    for B, Hkv, d, n, L in [(2, 2, 128, 1000, 64), (1, 3, 64, 700, 16), (2, 1, 128, 4096, 64), (1, 2, 128, 300, 3)]:
        data = rand_inputs(800 + n + d, B, Hkv, Hkv, d, n, "bf16")
        K = dev(data["K"])
        kc, k4 = host(csa.kv_cov_build(K, L)), host(csa.kv_cov4_build(K, L))
        torch.cuda.synchronize()
        shp = O.Shape(B, Hkv, Hkv, d, n, L, "bf16")
        assert np.array_equal(k4, O.cov4_pack(shp, kc)), f"Kcov4 differs (B={B} Hkv={Hkv} d={d} n={n} L={L})"


def cobs2_fp4_case(w, data, k=None, proxies=True):
    """GPU pipeline with FP4 second-order scores; the oracle decodes and scores the GPU's
    stored FP4 descriptors."""
    k = w.k if k is None else k
    q, K, V = dev(data["q"]), dev(data["K"]), dev(data["V"])
    Kbar, Vbar = csa.kv_summary_build(K, V, w.block_size)
    Kcov4 = csa.kv_cov4_build(K, w.block_size)
    scores = csa.block_score(q, Kcov4, "cobs2_fp4", w.block_size, n_tokens=w.n_tokens)
    sel = csa.topk_select(scores, k)
    out, lse = csa.sparse_decode_attn(q, K, V, Kbar, Vbar, sel, w.block_size, proxies=proxies)
    torch.cuda.synchronize()
    g = {"Kbar": host(Kbar), "Vbar": host(Vbar), "score": host(scores), "sel": host(sel), "out": host(out),
         "lse": host(lse)}
    shp = oshape(w, B=data["q"].shape[0], Hkv=data["K"].shape[1])
    Kbar_o, Vbar_o = O.kv_summary_build(shp, data["K"], data["V"])
    k4 = host(Kcov4)
    assert np.array_equal(k4[..., :2 * w.head_dim].copy().view(np.uint16), Kbar_o), "FP4 mean rows not bit-exact"
    score = O.group_score(shp, O.cobs2_fp4_logits(shp, data["q"], k4))
    sel_o, margin = O.topk_select(score, k)
    out_o, lse_o = O.sparse_decode_attn(shp, data["q"], data["K"], data["V"], Kbar_o, Vbar_o, sel_o, proxies)
    o = {"Kbar": Kbar_o, "Vbar": Vbar_o, "score": score, "sel": sel_o, "margin": margin, "out": out_o, "lse": lse_o}
    return g, o


@pytest.mark.parametrize("B,Hkv,G,n,L,k,d", [
    (2, 2, 4, 4096, 64, 5, 128),    # split scoring path (few KV heads)
    (8, 4, 4, 4096, 64, 5, 128),    # one workgroup per KV head
    (2, 2, 7, 3000, 64, 8, 128),    # G = 7, ragged last block
    (8, 4, 2, 2000, 32, 4, 64),     # d = 64, one workgroup per KV head, ragged
    (2, 2, 1, 1000, 16, 3, 64),     # d = 64, G = 1, split path
])
def test_cobs2_fp4_pipeline_matches_oracle(B, Hkv, G, n, L, k, d):
    w = W.Workload("cobs2_fp4_case", 0, B, G * Hkv, Hkv, d, n, L, "bf16", k, "cobs2_fp4", True, "clusters")
    data = rand_inputs(900 + B + G + n + d, B, G * Hkv, Hkv, d, n, "bf16")
    g, o = cobs2_fp4_case(w, data)
    compare_pipelines(w, g, o, f"cobs2 fp4 B={B} Hkv={Hkv} G={G} n={n} L={L} d={d}")


def test_cobs2_fp4_full_size_all_pairs():
    """The headline shape with FP4 second-order scores, as the benchmark runs it; the oracle
    scores every (b, KV head) pair from the stored FP4 descriptors."""
    w = W.WORKLOADS["llama3_8b_layer_b32_cobs2_fp4"]
    data = W.generate(w)
    g, o = cobs2_fp4_case(w, data)
    assert np.isfinite(g["out"]).all() and np.isfinite(g["lse"]).all()
    compare_pipelines(w, g, o, "cobs2 fp4 full size")


@pytest.mark.parametrize("mode", ["proxy_error", "cobs2_fp4", "box"])
@pytest.mark.parametrize("batch,n_kv_heads", [(2, 2), (8, 4)])  # split route, one workgroup per KV head
def test_descriptor_scores_replay_in_a_graph(mode, batch, n_kv_heads):
    """block_score over each descriptor captured in a HIP graph with topk_select and replayed
    several times, with eager work on the same buffers between replays: bit for bit the eager
    result each time."""
    w = small("llama3_8b_layer_b1", batch=batch, n_tokens=4096, n_kv_heads=n_kv_heads)
    data = W.generate(w)
    q, K = dev(data["q"]), dev(data["K"])
    build = {"proxy_error": csa.kv_var_build, "cobs2_fp4": csa.kv_cov4_build, "box": csa.kv_box_build}[mode]
    keys = build(K, w.block_size)
    shape = csa.make_shape(q, K, w.block_size)
    entry = {"proxy_error": csa.CSA_WS_BLOCK_SCORE_PROXY_ERROR, "cobs2_fp4": csa.CSA_WS_BLOCK_SCORE_COBS2_FP4,
             "box": csa.CSA_WS_BLOCK_SCORE_BOX}[mode]
    ws = torch.empty(max(1, csa.workspace_size(shape, entry)), dtype=torch.uint8, device="cuda")
    scores = torch.empty((w.batch, w.n_kv_heads, w.n_blocks), dtype=torch.float32, device="cuda")
    sel = torch.empty((w.batch, w.n_kv_heads, w.k), dtype=torch.int32, device="cuda")

    def run():
        csa.block_score(q, keys, mode, w.block_size, n_tokens=w.n_tokens, scores=scores, ws=ws)
        csa.topk_select(scores, w.k, sel=sel)

    run()
    torch.cuda.synchronize()
    ref = [host(scores).copy(), host(sel).copy()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        scores.fill_(float(i))
        sel.fill_(-1)
        ws.fill_(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(ref[0]), bits(host(scores))), f"{mode}: replay {i} scores"
        assert np.array_equal(ref[1], host(sel)), f"{mode}: replay {i} selection"


def test_cobs2_needs_bfloat16():
    w = W.WORKLOADS["tiny_f32_d64"]
    data = W.generate(w)
    Kcov = csa.kv_cov_build(dev(data["K"]), w.block_size)
    with pytest.raises(csa.CsaError, match="bfloat16"):
        csa.block_score(dev(data["q"]), Kcov, "cobs2", w.block_size, n_tokens=w.n_tokens)


def test_cobs2_full_size_all_pairs():
    """The headline shape with second-order scores, as the benchmark runs it; the oracle scores
    every (b, KV head) pair from the stored descriptors and checks one pair's descriptors
    against its own eigen-solve."""
    w = W.WORKLOADS["llama3_8b_layer_b32_cobs2"]
    data = W.generate(w)
    g, o = cobs2_case(w, data)
    assert np.isfinite(g["out"]).all() and np.isfinite(g["lse"]).all()
    compare_pipelines(w, g, o, "cobs2 full size")
    b, j = w.batch - 1, w.n_kv_heads - 1
    check_cov_descriptors(g["Kcov"][b:b + 1, j:j + 1], data["K"][b:b + 1, j:j + 1], oshape(w, B=1, Hkv=1),
                          f"pair ({b},{j})", 2e-2)


@pytest.mark.parametrize("fp4", [False, True], ids=["bf16", "fp4"])
def test_cobs2_end_to_end_selection_agreement(fp4):
    """Second-order ranking from the raw keys on both sides: the GPU builds its descriptors
    (fp32 eigen-solve, bfloat16 or FP4 storage) and ranks with them; the oracle builds its own
    (fp64 eigen-solve, the same storage) and ranks with those.  Eigenvectors differ in their
    last bits, so the selections are compared as a whole: the fraction of (b, KV head) rows that
    agree is reported, and a row may disagree only where the score change that the descriptor
    difference itself causes (the oracle's scores from the GPU's descriptors against those from
    its own) reaches the row's margin."""
    w = small("llama3_8b_layer_b32_cobs2", batch=4, n_tokens=4096)  # 32 rows of 64 blocks
    data = W.generate(w)
    shp = oshape(w)
    q, K = dev(data["q"]), dev(data["K"])
    mode = "cobs2_fp4" if fp4 else "cobs2"
    desc = (csa.kv_cov4_build if fp4 else csa.kv_cov_build)(K, w.block_size)
    sel_g = host(csa.topk_select(csa.block_score(q, desc, mode, w.block_size, n_tokens=w.n_tokens), w.k))
    torch.cuda.synchronize()
    desc_g = host(desc)
    desc_o = O.cov_build(shp, data["K"])
    if fp4:
        desc_o = O.cov4_pack(shp, desc_o)
    logits = O.cobs2_fp4_logits if fp4 else O.cobs2_logits
    score_o = O.group_score(shp, logits(shp, data["q"], desc_o))
    score_x = O.group_score(shp, logits(shp, data["q"], desc_g))
    sel_o, margin = O.topk_select(score_o, w.k)
    rows = sel_o.shape[0] * sel_o.shape[1]
    sel_o, sel_g = sel_o.reshape(rows, -1), sel_g.reshape(rows, -1)
    pert = np.abs(score_x - score_o).reshape(rows, -1).max(axis=1)
    kth = -np.sort(-score_o.reshape(rows, -1), axis=1)[:, w.k - 1]
    margin = margin.reshape(-1)
    differ = [r for r in range(rows) if not np.array_equal(sel_o[r], sel_g[r])]
    parity_report.note(f"second-order ranking end to end ({mode}, descriptors built on each side): "
                       f"{rows - len(differ)} of {rows} rows select the same blocks")
    for r in differ:
        parity_report.note(f"  row {r}: margin {margin[r]:.3e}, score change from the descriptor difference "
                           f"{pert[r]:.3e}")
        assert margin[r] <= 2 * pert[r] + 2 * score_bound(kth[r]), \
            f"{mode}: row {r} disagrees with margin {margin[r]:.3e} beyond the descriptor change {pert[r]:.3e}"
    assert len(differ) <= rows // 4, f"{mode}: {len(differ)} of {rows} rows disagree"


@pytest.mark.parametrize("mode", ["summary", "exact_mass"])
def test_largest_group_and_long_context(mode):
    """Edge of the supported sizes: one sequence with a 64-head group over a 1M-token cache
    (256 MiB per tensor: 32-bit buffer offsets near their top), 16384 blocks (the radix top-k),
    k = 32, proxies for the rest, fully checked against the oracle."""
    n, G, d, L, k = 1 << 20, 64, 128, 64, 32
    w = W.Workload("max_case", 0, 1, G, 1, d, n, L, "bf16", k, mode, True, "clusters")
    data = rand_inputs(400, 1, G, 1, d, n, "bf16", qscale=3.0)
    compare_pipelines(w, gpu_pipeline(w, data), oracle_pipeline(w, data), f"max case {mode}")


# ---------------------------------------------------------------------------
# proxy-error ranking (mean and variance tokens)
# ---------------------------------------------------------------------------

VAR_CASES = [
    ("f32_d64_L16", W.Workload("v", 0, 1, 2, 2, 64, 700, 16, "f32", 3, "proxy_error", True, "clusters")),
    ("bf16_d128_ragged", W.Workload("v", 0, 2, 4, 2, 128, 1000, 64, "bf16", 3, "proxy_error", True, "clusters")),
    ("bf16_d64_L1", W.Workload("v", 0, 1, 2, 1, 64, 256, 1, "bf16", 3, "proxy_error", True, "clusters")),
    ("bf16_d128_L48", W.Workload("v", 0, 1, 2, 2, 128, 2000, 48, "bf16", 3, "proxy_error", True, "clusters")),
]


@pytest.mark.parametrize("name,w", VAR_CASES, ids=[c[0] for c in VAR_CASES])
def test_var_tokens_match_oracle_bit_for_bit(name, w):
    data = rand_inputs(500 + w.n_tokens, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_tokens, w.dtype)
    kv = host(csa.kv_var_build(dev(data["K"]), w.block_size))
    torch.cuda.synchronize()
    ko = O.var_build(oshape(w), data["K"])
    assert np.array_equal(bits(kv), bits(ko)), f"{name}: Kvar not bit-exact"


@pytest.mark.parametrize("B,Hkv,G,n,L,k", [
    (2, 2, 4, 4096, 64, 5),     # split scoring path (few KV heads)
    (8, 4, 4, 4096, 64, 5),     # one workgroup per KV head
    (2, 2, 7, 3000, 64, 8),     # G = 7, ragged last block
    (2, 2, 1, 2048, 32, 3),     # one head per KV head
    (8, 4, 2, 1000, 16, 4),     # one workgroup per KV head, ragged, G = 2
])
def test_proxy_error_pipeline_matches_oracle(B, Hkv, G, n, L, k):
    w = W.Workload("err_case", 0, B, G * Hkv, Hkv, 128, n, L, "bf16", k, "proxy_error", True, "clusters")
    data = rand_inputs(600 + B + G + n, B, G * Hkv, Hkv, 128, n, "bf16")
    compare_pipelines(w, gpu_pipeline(w, data), oracle_pipeline(w, data), f"proxy error B={B} Hkv={Hkv} G={G}")


@pytest.mark.parametrize("B,Hkv,G,n,L,k", [
    (8, 4, 4, 2048, 32, 4),     # d = 64, one workgroup per KV head
    (2, 2, 2, 1000, 16, 3),     # d = 64, split kernels, ragged
])
def test_proxy_error_pipeline_d64_matches_oracle(B, Hkv, G, n, L, k):
    """The proxy-error kernels at d = 64 (eight lanes per mean or variance row in their loads)."""
    w = W.Workload("err_d64", 0, B, G * Hkv, Hkv, 64, n, L, "bf16", k, "proxy_error", True, "clusters")
    data = rand_inputs(610 + B + G + n, B, G * Hkv, Hkv, 64, n, "bf16")
    compare_pipelines(w, gpu_pipeline(w, data), oracle_pipeline(w, data), f"proxy error d=64 B={B} Hkv={Hkv} G={G}")


@pytest.mark.parametrize("B,Hkv", [(1, 2), (8, 4)])
def test_proxy_error_exact_proxies_score_minus_infinity(B, Hkv):
    """Blocks of equal keys leave no error: -inf on both sides, never selected before the
    others, through both scoring routes."""
    G, n, L, k = 4, 2048, 64, 4
    w = W.Workload("err_eq", 0, B, G * Hkv, Hkv, 128, n, L, "bf16", k, "proxy_error", True, "clusters")
    data = rand_inputs(700 + B, B, G * Hkv, Hkv, 128, n, "bf16")
    for blk in (0, 3, 31):
        data["K"][:, :, blk * L:(blk + 1) * L] = data["K"][:, :, blk * L:blk * L + 1]
    g, o = gpu_pipeline(w, data), oracle_pipeline(w, data)
    assert np.all(g["score"][:, :, [0, 3, 31]] == -np.inf)
    assert np.isfinite(np.delete(g["score"], [0, 3, 31], axis=2)).all()
    compare_pipelines(w, g, o, f"proxy error, equal-key blocks, B={B}")


def test_proxy_error_needs_bfloat16():
    w = W.WORKLOADS["tiny_f32_d64"]
    data = W.generate(w)
    Kvar = csa.kv_var_build(dev(data["K"]), w.block_size)
    with pytest.raises(csa.CsaError, match="bfloat16"):
        csa.block_score(dev(data["q"]), Kvar, "proxy_error", w.block_size, n_tokens=w.n_tokens)
