"""Host logic of bench.py (no GPU): byte accounting, the route label, the source hash that
guards the stored HBM traffic, and the refusal of several GPUs."""
import os
import shutil
import subprocess
import sys

import bench
from coreset_softmax_attention_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_headline_byte_counts():
    """Per (sequence, KV head) of the 32-sequence layer: exact K+V 5 x 64 x 2 x 256 B, the other
    507 blocks' mean key and value rows 507 x 2 x 256 B, q 4 x 256 B, the selection 5 x 4 B;
    written: 4 heads x (128 + 1) fp32.  Times 256 pairs.  The one-kernel step reads all 512
    mean keys (the five selected ones too) and no selection."""
    w = W.WORKLOADS["llama3_8b_layer_b32"]
    rd, wr = bench.algorithmic_bytes(w)
    assert (rd, wr) == (256 * (163840 + 259584 + 1024 + 20), 256 * 4 * 129 * 4)
    assert (rd, wr) == (108_663_808, 528_384)
    srd, swr = bench.step_bytes(w)
    assert srd == 256 * (512 * 256 + 507 * 256 + 5 * 64 * 2 * 256 + 1024) and swr == wr
    assert srd + swr == 109_514_752


def test_weighted_tokens_add_their_rows():
    w = W.WORKLOADS["weighted_coreset_128k"]
    rd0, _ = bench.step_bytes(w)
    rd1, _ = bench.step_bytes(w, m=w.coreset)
    assert rd1 - rd0 == w.batch * w.n_kv_heads * w.coreset * (2 * w.head_dim * 2 + 8)


def test_route_label_follows_the_step_rule():
    one, split, ranked = "decode_step_kernel", "in turn", "ranking the candidates"
    assert one in bench.step_kernels(W.WORKLOADS["llama3_8b_layer_b32"])   # 256 KV heads
    assert one in bench.step_kernels(W.WORKLOADS["llama3_8b_layer_b1"])    # 8, small share each
    assert ranked in bench.step_kernels(W.WORKLOADS["weighted_coreset_128k"])  # 16 KV heads, 2048 blocks
    assert split in bench.step_kernels(W.WORKLOADS["exact_mass_gqa_b8"])   # exact-mass scores
    # a small share over more than 512 blocks takes the split kernels
    assert ranked in bench.step_kernels(W.WORKLOADS["llama3_8b_layer_b1"].with_(n_tokens=40000, proxies=False))


def test_source_hash_ignores_comments_but_not_code(tmp_path):
    src = os.path.join(ROOT, "coreset_softmax_attention_amd", "csrc")
    dst = tmp_path / "csrc"
    shutil.copytree(src, dst)
    h0 = bench.source_hash(str(dst))
    assert h0 == bench.source_hash()
    f = dst / "launch.hpp"
    text = f.read_text()
    f.write_text("// a comment line\n" + text.replace("\n", "\n  ", 3) + "/* block\n comment */\n")
    assert bench.source_hash(str(dst)) == h0
    f.write_text(text.replace("kFusedStepSmallWork = 4096", "kFusedStepSmallWork = 4097"))
    assert bench.source_hash(str(dst)) != h0


def test_several_gpus_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_timing_detail_counts_what_was_timed():
    class A:
        steps, windows = 20, 15

    d = bench.timing_detail(A, {"step": [0.025 + 0.001 * i for i in range(15)]})
    assert d["timed_launches_per_window"] == 20 and d["windows"] == 15 and d["timed_launches"] == 300
    assert abs(d["step_us"]["median"] - 32.0) < 1e-9 and d["step_us"]["min"] == 25.0
    assert bench.timing_detail(A, None) == {"mode": "eager", "timed_launches": 20, "windows": 1}


def test_cpu_model_names_family_and_affinity():
    s = bench.cpu_model()
    assert "family" in s and "logical CPUs" in s


def test_cluster_bytes_counts_the_selection_actually_made():
    """Two KV heads, four clusters of sizes (3, 0, 5, 2) and (1, 1, 1, 7), top-2 read exactly: the
    step reads every mean key, the mean values of the unread non-empty clusters and the exact
    rows of the selected ones; the attention kernel reads both mean rows of the unread ones."""
    import json

    import numpy as np

    import bench
    from coreset_softmax_attention_amd import workloads as W

    w = W.WORKLOADS["llama3_8b_layer_b32_qgc"].with_(batch=1, n_q_heads=4, n_kv_heads=2, qgc=4, k=2)
    sizes = np.array([[[3, 0, 5, 2], [1, 1, 1, 7]]])
    sel = np.array([[[0, 2], [1, 3]]])
    by = bench.cluster_bytes(w, sizes, sel)
    row = 128 * 2
    assert by["exact_tokens"] == 3 + 5 + 1 + 7
    assert by["unread_clusters"] == 1 + 2  # cluster 3 of head 0; clusters 0 and 2 of head 1
    common = 2 * (5 * 4 + 2 * row + 4 * 2) + 16 * 2 * row
    assert by["step"] == (common + 2 * 4 * row + 3 * row, 2 * 2 * 129 * 4)
    assert by["attn"] == (common + 3 * 2 * row, 2 * 2 * 129 * 4)
    json.dumps(by)


def test_kernel_source_hash_follows_only_its_own_files(tmp_path):
    """A kernel's traffic stays valid when another kernel's source or a host declaration
    changes, and goes stale when its own source or a shared device header does."""
    src = os.path.join(ROOT, "coreset_softmax_attention_amd", "csrc")
    dst = tmp_path / "csrc"
    shutil.copytree(src, dst)
    files = bench.KERNEL_SOURCES["decode_step"]
    h0 = bench.source_hash(str(dst), files)
    for other in ("cluster.hip", "launch.hpp"):
        f = dst / other
        f.write_text(f.read_text() + "\nstatic int unused_marker = 1;\n")
    assert bench.source_hash(str(dst), files) == h0
    for own in ("step.hip", "attn_engine.hpp"):
        f = dst / own
        text = f.read_text()
        f.write_text(text + "\nstatic int unused_marker = 1;\n")
        assert bench.source_hash(str(dst), files) != h0
        f.write_text(text)
    assert bench.source_hash(str(dst), files) == h0


def test_three_call_traffic_sums_the_route_kernels():
    """The step traffic of the three-call route is the sum of its kernels' measured bytes per
    launch, and null when the score kernel, the top-k or the attention is missing (not
    measured, or measured on other sources)."""
    t = {"block_score_cobs2_split": 100.0, "score_finish": 10.0, "topk": 1.0, "sparse_decode_attn": 1000.0,
         "decode_step": 5.0}
    assert bench.three_call_traffic(t) == 1111.0
    assert bench.three_call_traffic({"block_score_box": 7.0, "topk": 1.0, "sparse_decode_attn": 2.0}) == 10.0
    for drop in ("block_score_cobs2_split", "topk", "sparse_decode_attn"):
        assert bench.three_call_traffic({k: v for k, v in t.items() if k != drop}) is None
    assert bench.three_call_traffic(None) is None
    # every counted kernel has its device sources listed
    assert set(bench.TRAFFIC_KERNELS) == set(bench.KERNEL_SOURCES)
    assert set(bench.THREE_CALL_KERNELS) <= set(bench.TRAFFIC_KERNELS)
