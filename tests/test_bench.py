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
    one, split = "decode_step_kernel", "in turn"
    assert one in bench.step_kernels(W.WORKLOADS["llama3_8b_layer_b32"])   # 256 KV heads
    assert one in bench.step_kernels(W.WORKLOADS["llama3_8b_layer_b1"])    # 8, small share each
    assert split in bench.step_kernels(W.WORKLOADS["weighted_coreset_128k"])  # (2040+512+2048) x 7
    assert split in bench.step_kernels(W.WORKLOADS["exact_mass_gqa_b8"])   # exact-mass scores


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
