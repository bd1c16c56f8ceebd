"""selective_decode_step_noalloc through the C-ABI: the decode step with the library's static
per-GPU scratch instead of a caller workspace.  Two calls in a row on shapes that take the
three-kernel route (which needs scratch), the second smaller than the first, each against
selective_decode_step with a workspace (bit for bit: the same kernels on the same inputs) and
against the oracle (summaries and selections bit for bit, outputs per row within 2e-3).  Runs
alone in a fresh process and after the other GPU tests (the buffer keeps the previous call's
contents; nothing in it needs to start at zero)."""
import ctypes

import numpy as np
import pytest
import torch

from coreset_softmax_attention_amd import csa
from coreset_softmax_attention_amd import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def noalloc_step(w, q, K, V, Kbar, Vbar, ti, tw):
    dev = q.device
    B, Hq, d = q.shape
    nb, k, m = w.n_blocks, min(w.k, w.n_blocks), w.coreset
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
    scores = torch.full((B, w.n_kv_heads, nb), float("nan"), dtype=torch.float32, device=dev)
    sel = torch.full((B, w.n_kv_heads, k), -1, dtype=torch.int32, device=dev)
    shape = csa.make_shape(q, K, w.block_size)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    rc = csa.lib().selective_decode_step_noalloc(
        ctypes.byref(shape), csa.MODES[w.score_mode], p(q), p(K), p(V), p(Kbar), p(Vbar), k, p(ti), p(tw), m,
        csa.CSA_PROXY_COMPLEMENT if w.proxies else csa.CSA_PROXY_NONE, p(scores), p(sel), p(out), p(lse),
        ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert rc == csa.CSA_OK, csa.lib().csa_last_error()
    return out, lse, scores, sel


# the three-kernel route (few KV heads, a large share each: (proxies + k L + m) G > 4096)
CASES = [
    W.scaled_down(W.WORKLOADS["weighted_coreset_128k"], batch=2, n_tokens=16384, n_kv_heads=2)
    .with_(coreset=600),
    W.scaled_down(W.WORKLOADS["weighted_coreset_128k"], batch=1, n_tokens=8192, n_kv_heads=2).with_(coreset=300),
]


# the split route beyond 512 blocks (chunk candidates ranked by the attention kernel), whose
# candidates also live in the scratch
RANKED_CASES = [
    W.scaled_down(W.WORKLOADS["weighted_coreset_128k"], batch=1, n_tokens=65536, n_kv_heads=2).with_(coreset=300),
    W.scaled_down(W.WORKLOADS["weighted_coreset_128k"], batch=1, n_tokens=40960, n_kv_heads=2).with_(coreset=200),
]


def test_noalloc_step_matches_the_step_with_a_workspace_twice_in_a_row():
    check_twice(CASES)


def test_noalloc_ranked_route_matches_the_step_with_a_workspace_twice_in_a_row():
    assert all(w.n_blocks > 512 for w in RANKED_CASES)
    check_twice(RANKED_CASES)


def check_twice(cases):
    shape0 = csa.Shape(cases[0].batch, cases[0].n_q_heads, cases[0].n_kv_heads, cases[0].head_dim,
                       cases[0].n_tokens, cases[0].block_size, csa.CSA_BF16, 0.0)
    need = csa.lib().csa_workspace_size(ctypes.byref(shape0), csa.CSA_WS_SELECTIVE_DECODE_STEP, cases[0].k,
                                        cases[0].coreset)
    assert 0 < need <= csa.CSA_STEP_NOALLOC_SCRATCH_BYTES  # this route does use the scratch
    for i, w in enumerate(cases):
        print(f"noalloc call {i}: B={w.batch} Hkv={w.n_kv_heads} n={w.n_tokens} m={w.coreset}", flush=True)
        data = W.generate(w)
        q, K, V = (csa.to_device(data[x]) for x in ("q", "K", "V"))
        ti, tw = csa.to_device(data["tok_idx"]), csa.to_device(data["tok_logw"])
        Kbar, Vbar = csa.kv_summary_build(K, V, w.block_size)
        got = noalloc_step(w, q, K, V, Kbar, Vbar, ti, tw)
        ref = csa.selective_decode_step(q, K, V, Kbar, Vbar, w.k, w.block_size, mode=w.score_mode,
                                        proxies=w.proxies, tok_idx=ti, tok_logw=tw, want_scores=True, want_sel=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "scores", "sel"), got, ref):
            assert np.array_equal(bits(host(a)), bits(host(b))), f"call {i}: {name} differs from the workspace route"
        # against the oracle
        shp = O.Shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_tokens, w.block_size, w.dtype)
        Kb_o, Vb_o = O.kv_summary_build(shp, data["K"], data["V"])
        assert np.array_equal(host(Kbar), Kb_o) and np.array_equal(host(Vbar), Vb_o)
        score = O.block_score(shp, O.SUMMARY, data["q"], Kb_o)
        sel_o, margin = O.topk_select(score, w.k)
        out_o, lse_o = O.sparse_decode_attn(shp, data["q"], data["K"], data["V"], Kb_o, Vb_o, sel_o, True,
                                            data["tok_idx"], data["tok_logw"])
        assert np.array_equal(host(got[3]), sel_o), f"call {i}: selection differs from the oracle"
        o = host(got[0]).astype(np.float64)
        err = (np.abs(o - out_o).max(axis=-1) / np.abs(out_o).max(axis=-1)).max()
        assert err <= 2e-3, f"call {i}: output row error {err:.3e}"
        assert np.abs(host(got[1]) - lse_o).max() <= 1e-3
