"""The C-ABI library without a GPU: it loads, exports every function include/csa.h
declares, and rejects invalid arguments on the host before launching anything.
No call here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

from coreset_softmax_attention_amd import csa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")
FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced (validation fails first)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(csa.library_path()):
        from coreset_softmax_attention_amd import build_lib

        build_lib.build()
    return csa.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_entry_points():
    names = set(declared_functions())
    assert {"kv_summary_build", "kv_box_build", "kv_cov_build", "kv_cov4_build", "kv_var_build", "block_score", "topk_select", "sparse_decode_attn",
            "dense_decode_attn", "selective_decode_step", "csa_workspace_size", "csa_status_str",
            "csa_last_error"} <= names


def test_library_exports_every_declared_function(L):
    out = subprocess.run(["nm", "-D", "--defined-only", csa.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_header_is_valid_c():
    subprocess.run(["gcc", "-x", "c", "-std=c11", "-fsyntax-only", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", HEADER], check=True)


def shape(B=2, Hq=8, Hkv=2, d=128, n=1024, L=64, dtype=csa.CSA_BF16, scale=0.0):
    return csa.Shape(B, Hq, Hkv, d, n, L, dtype, scale)


def sparse(L, s, k=2, m=0, proxy=1, sel=FAKE, ptrs=FAKE, ws=None, wsb=0, kbar=FAKE):
    p = ptrs
    return L.sparse_decode_attn(ctypes.byref(s) if s is not None else None, p, p, p, kbar, kbar, sel, k,
                                FAKE if m else None, FAKE if m else None, m, proxy, p, p, ws, wsb, None)


def test_status_strings(L):
    assert L.csa_status_str(0) == b"ok"
    assert L.csa_status_str(-1) == b"invalid argument"
    assert L.csa_status_str(-2) == b"unsupported"
    assert L.csa_status_str(-3) == b"workspace missing or too small"
    assert L.csa_status_str(-4) == b"HIP error"


@pytest.mark.parametrize("bad,code,msg", [
    (dict(B=0), csa.CSA_ERR_INVALID_ARG, b"non-positive"),
    (dict(Hq=6, Hkv=4), csa.CSA_ERR_INVALID_ARG, b"multiple"),
    (dict(d=96), csa.CSA_ERR_UNSUPPORTED, b"head_dim 96"),
    (dict(dtype=7), csa.CSA_ERR_INVALID_ARG, b"dtype"),
    (dict(scale=float("inf")), csa.CSA_ERR_INVALID_ARG, b"scale"),
    (dict(Hq=130, Hkv=2), csa.CSA_ERR_UNSUPPORTED, b"group size"),
])
def test_shape_validation(L, bad, code, msg):
    s = shape(**bad)
    assert sparse(L, s) == code
    assert msg in L.csa_last_error()
    assert L.dense_decode_attn(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == code
    assert L.kv_summary_build(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None) == code
    assert L.kv_box_build(ctypes.byref(s), FAKE, FAKE, None) == code
    assert L.block_score(ctypes.byref(s), 0, FAKE, FAKE, FAKE, None, 0, None) == code
    assert L.block_score(ctypes.byref(s), 2, FAKE, FAKE, FAKE, None, 0, None) == code
    assert L.csa_workspace_size(ctypes.byref(s), 2, 1, 0) == 0


def test_null_shape(L):
    assert sparse(L, None) == csa.CSA_ERR_INVALID_ARG
    assert b"shape is NULL" in L.csa_last_error()


def test_sparse_argument_checks(L):
    s = shape()  # nb = 16
    assert sparse(L, s, k=0, m=0, proxy=0) == csa.CSA_ERR_INVALID_ARG
    assert b"empty virtual-token set" in L.csa_last_error()
    assert sparse(L, s, k=17) == csa.CSA_ERR_INVALID_ARG
    assert sparse(L, s, k=-1) == csa.CSA_ERR_INVALID_ARG
    assert sparse(L, s, k=2, sel=None) == csa.CSA_ERR_INVALID_ARG
    assert sparse(L, s, proxy=5) == csa.CSA_ERR_INVALID_ARG
    assert sparse(L, s, proxy=1, kbar=None) == csa.CSA_ERR_INVALID_ARG
    assert sparse(L, s, ptrs=FAKE + 2) == csa.CSA_ERR_INVALID_ARG
    assert b"misaligned" in L.csa_last_error()
    m_bad = L.sparse_decode_attn(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, None, None, 3, 1, FAKE,
                                 FAKE, None, 0, None)
    assert m_bad == csa.CSA_ERR_INVALID_ARG and b"weighted tokens missing" in L.csa_last_error()


def test_workspace_is_checked_before_launch(L):
    s = shape(B=1, Hq=32, Hkv=8, n=32768)  # one sequence: split-K partials need a workspace
    need = L.csa_workspace_size(ctypes.byref(s), csa.CSA_WS_SPARSE_DECODE_ATTN, 5, 0)
    assert need > 0
    assert sparse(L, s, k=5, ws=None) == csa.CSA_ERR_WORKSPACE
    assert sparse(L, s, k=5, ws=FAKE, wsb=need - 1) == csa.CSA_ERR_WORKSPACE
    assert sparse(L, s, k=5, ws=FAKE + 8, wsb=need) == csa.CSA_ERR_WORKSPACE
    assert sparse(L, s, k=5, ws=FAKE + 128, wsb=need) == csa.CSA_ERR_WORKSPACE  # 16- but not 256-aligned
    assert b"256-byte" in L.csa_last_error()
    dneed = L.csa_workspace_size(ctypes.byref(s), csa.CSA_WS_DENSE_DECODE_ATTN, 0, 0)
    assert dneed > 0
    assert L.dense_decode_attn(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == csa.CSA_ERR_WORKSPACE
    bneed = L.csa_workspace_size(ctypes.byref(s), csa.CSA_WS_BLOCK_SCORE_SUMMARY, 0, 0)
    # logits [B, Hq, nb], 256-byte aligned, then (max, sum) per (KV head, tile of 32 blocks, 8 heads)
    assert bneed == 1 * 32 * 512 * 4 + 8 * 16 * 16 * 4
    assert L.block_score(ctypes.byref(s), 0, FAKE, FAKE, FAKE, None, 0, None) == csa.CSA_ERR_WORKSPACE
    assert L.block_score(ctypes.byref(s), 9, FAKE, FAKE, FAKE, None, 0, None) == csa.CSA_ERR_INVALID_ARG
    assert L.csa_workspace_size(ctypes.byref(s), csa.CSA_WS_BLOCK_SCORE_BOX, 0, 0) == bneed
    assert L.block_score(ctypes.byref(s), csa.CSA_SCORE_BOX, FAKE, FAKE, FAKE, None, 0, None) == csa.CSA_ERR_WORKSPACE


def test_cov_build_argument_checks(L):
    s = shape()
    assert L.kv_cov_build(ctypes.byref(s), None, FAKE, None) == csa.CSA_ERR_INVALID_ARG
    assert L.kv_cov_build(ctypes.byref(s), FAKE, FAKE + 4, None) == csa.CSA_ERR_INVALID_ARG
    big = shape(L=128)
    assert L.kv_cov_build(ctypes.byref(big), FAKE, FAKE, None) == csa.CSA_ERR_UNSUPPORTED
    assert b"at most 64" in L.csa_last_error()
    f32 = shape(dtype=csa.CSA_F32)
    assert L.block_score(ctypes.byref(f32), csa.CSA_SCORE_COBS2, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                         None) == csa.CSA_ERR_UNSUPPORTED
    assert step(L, s, mode=csa.CSA_SCORE_COBS2) == csa.CSA_ERR_UNSUPPORTED


def test_var_build_and_proxy_error_argument_checks(L):
    s = shape()  # B=2, Hq=8, Hkv=2, n=1024, L=64: nb = 16, one tile of 32 blocks per KV head
    assert L.kv_var_build(ctypes.byref(s), None, FAKE, None) == csa.CSA_ERR_INVALID_ARG
    assert L.kv_var_build(ctypes.byref(s), FAKE, FAKE + 8, None) == csa.CSA_ERR_INVALID_ARG
    assert b"aligned" in L.csa_last_error()
    assert L.kv_var_build(None, FAKE, FAKE, None) == csa.CSA_ERR_INVALID_ARG
    # log-errors [B, Hq, nb], 256-byte aligned, then (max, sum) per (KV head, tile, 8 heads)
    need = L.csa_workspace_size(ctypes.byref(s), csa.CSA_WS_BLOCK_SCORE_PROXY_ERROR, 0, 0)
    assert need == 2 * 8 * 16 * 4 + 2 * 2 * 1 * 16 * 4
    assert L.block_score(ctypes.byref(s), csa.CSA_SCORE_PROXY_ERROR, FAKE, FAKE, FAKE, None, 0,
                         None) == csa.CSA_ERR_WORKSPACE
    g1 = shape(Hq=2)
    assert L.csa_workspace_size(ctypes.byref(g1), csa.CSA_WS_BLOCK_SCORE_PROXY_ERROR, 0, 0) == 0
    f32 = shape(dtype=csa.CSA_F32)
    assert L.block_score(ctypes.byref(f32), csa.CSA_SCORE_PROXY_ERROR, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                         None) == csa.CSA_ERR_UNSUPPORTED
    assert b"proxy-error" in L.csa_last_error()
    assert step(L, s, mode=csa.CSA_SCORE_PROXY_ERROR) == csa.CSA_ERR_UNSUPPORTED


def test_cov4_build_argument_checks(L):
    s = shape()
    assert L.kv_cov4_build(ctypes.byref(s), None, FAKE, None) == csa.CSA_ERR_INVALID_ARG
    assert L.kv_cov4_build(ctypes.byref(s), FAKE, FAKE + 4, None) == csa.CSA_ERR_INVALID_ARG
    assert L.kv_cov4_build(ctypes.byref(shape(L=128)), FAKE, FAKE, None) == csa.CSA_ERR_UNSUPPORTED
    assert L.kv_cov4_build(ctypes.byref(shape(dtype=csa.CSA_F32)), FAKE, FAKE, None) == csa.CSA_ERR_UNSUPPORTED
    assert b"bfloat16" in L.csa_last_error()
    assert csa.cov4_block_bytes(128) == 256 + 16 + 256  # mean, scales, codes: the factor is 272 bytes
    assert L.csa_workspace_size(ctypes.byref(s), csa.CSA_WS_BLOCK_SCORE_COBS2_FP4, 0, 0) == \
        L.csa_workspace_size(ctypes.byref(s), csa.CSA_WS_BLOCK_SCORE_COBS2, 0, 0)
    assert L.block_score(ctypes.byref(shape(dtype=csa.CSA_F32)), csa.CSA_SCORE_COBS2_FP4, FAKE, FAKE, FAKE, FAKE,
                         1 << 20, None) == csa.CSA_ERR_UNSUPPORTED
    assert step(L, s, mode=csa.CSA_SCORE_COBS2_FP4) == csa.CSA_ERR_UNSUPPORTED


def test_box_build_argument_checks(L):
    s = shape()
    assert L.kv_box_build(ctypes.byref(s), None, FAKE, None) == csa.CSA_ERR_INVALID_ARG
    assert L.kv_box_build(ctypes.byref(s), FAKE, FAKE + 8, None) == csa.CSA_ERR_INVALID_ARG
    assert b"aligned" in L.csa_last_error()
    assert L.kv_box_build(None, FAKE, FAKE, None) == csa.CSA_ERR_INVALID_ARG


def test_workspace_size_with_no_exact_or_weighted_tokens(L):
    s = shape()
    assert L.csa_workspace_size(ctypes.byref(s), csa.CSA_WS_SPARSE_DECODE_ATTN, 0, 0) >= 0


def test_workspace_sizes(L):
    mha = shape(B=8, Hq=32, Hkv=32, n=32768)
    assert L.csa_workspace_size(ctypes.byref(mha), csa.CSA_WS_BLOCK_SCORE_EXACT_MASS, 0, 0) == 0  # G = 1
    assert L.csa_workspace_size(ctypes.byref(mha), 17, 0, 0) == 0
    assert b"unknown entry" in L.csa_last_error()
    assert L.csa_workspace_size(ctypes.byref(mha), csa.CSA_WS_SPARSE_DECODE_ATTN, 513, 0) == 0


def test_topk_argument_checks(L):
    assert L.topk_select(-1, 4, 2, FAKE, FAKE, None) == csa.CSA_ERR_INVALID_ARG
    assert L.topk_select(3, 0, 2, FAKE, FAKE, None) == csa.CSA_ERR_INVALID_ARG
    assert L.topk_select(3, 4, -2, FAKE, FAKE, None) == csa.CSA_ERR_INVALID_ARG
    assert L.topk_select(3, 4, 2, None, FAKE, None) == csa.CSA_ERR_INVALID_ARG
    assert L.topk_select(3, 4, 2, FAKE + 1, FAKE, None) == csa.CSA_ERR_INVALID_ARG
    # nothing to do: no launch, OK
    assert L.topk_select(0, 4, 2, None, None, None) == csa.CSA_OK
    assert L.topk_select(3, 4, 0, None, None, None) == csa.CSA_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(csa, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(csa, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        csa.lib()


def step(L, s, mode=0, k=2, m=0, proxy=1, ptrs=FAKE, kbar=FAKE, ws=None, wsb=0):
    p = ptrs
    return L.selective_decode_step(ctypes.byref(s) if s is not None else None, mode, p, p, p, kbar, kbar, k,
                                   FAKE if m else None, FAKE if m else None, m, proxy, None, None, p, p, ws, wsb,
                                   None)


def test_decode_step_argument_checks(L):
    s = shape()
    assert step(L, None) == csa.CSA_ERR_INVALID_ARG
    assert step(L, s, mode=9) == csa.CSA_ERR_INVALID_ARG
    assert step(L, s, mode=csa.CSA_SCORE_BOX) == csa.CSA_ERR_UNSUPPORTED
    assert b"Kbox" in L.csa_last_error()
    assert step(L, s, proxy=3) == csa.CSA_ERR_INVALID_ARG
    assert step(L, s, k=0, proxy=0) == csa.CSA_ERR_INVALID_ARG
    assert b"empty virtual-token set" in L.csa_last_error()
    assert step(L, s, k=-1) == csa.CSA_ERR_INVALID_ARG
    assert step(L, s, kbar=None) == csa.CSA_ERR_INVALID_ARG
    assert step(L, s, ptrs=FAKE + 4) == csa.CSA_ERR_INVALID_ARG
    assert step(L, shape(d=80)) == csa.CSA_ERR_UNSUPPORTED
    # a shape the one-kernel path does not take (B * Hkv < 32 and a large share per KV head:
    # (1022 proxies + 2 x 64 exact rows) x 4 heads > 4096) needs the workspace
    big = shape(n=65536)
    need = L.csa_workspace_size(ctypes.byref(big), csa.CSA_WS_SELECTIVE_DECODE_STEP, 2, 0)
    assert need >= 2 * 2 * 1024 * 4
    assert step(L, big, ws=None) == csa.CSA_ERR_WORKSPACE
    assert step(L, big, ws=FAKE, wsb=need - 1) == csa.CSA_ERR_WORKSPACE


def test_block_score_rejects_keys_of_4_gib_per_kv_head(L):
    """The scoring kernels address one KV head's key rows with 32-bit offsets."""
    big_exact = shape(B=1, Hq=2, Hkv=1, n=1 << 24)  # 2^24 tokens x 256 B
    assert L.block_score(ctypes.byref(big_exact), csa.CSA_SCORE_EXACT_MASS, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                         None) == csa.CSA_ERR_UNSUPPORTED
    assert b"4 GiB" in L.csa_last_error()
    big_box = shape(B=1, Hq=2, Hkv=1, n=1 << 23, L=1)  # 2^23 blocks x 2 rows x 256 B
    assert L.block_score(ctypes.byref(big_box), csa.CSA_SCORE_BOX, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                         None) == csa.CSA_ERR_UNSUPPORTED


def test_kernels_fit_their_registers(L):
    """No kernel spills to scratch memory (a spill in a streaming kernel costs more than its
    loads), eight query heads per KV head included; the decode-step and attention kernels of
    four and of eight heads (over blocks and over clusters) run two waves per SIMD.  Figures from the compiler's resource
    report, written when the library is built."""
    import json
    from coreset_softmax_attention_amd import build_lib

    if not os.path.exists(build_lib.RESOURCES) or (os.path.getmtime(build_lib.RESOURCES) <
                                                    os.path.getmtime(csa.library_path()) - 60):
        build_lib.build()
    res = json.load(open(build_lib.RESOURCES))
    assert len(res) > 100, "resource report incomplete"
    for name, r in res.items():
        assert r.get("scratch_bytes_per_lane", 0) == 0 and r.get("vgpr_spills", 0) == 0, f"{name} spills: {r}"
    for part in ("decode_step_kernelILi128ELi4ELb0E", "attn_mfma_kernelILi128ELi4ELi8E",
                 "decode_step_kernelILi128ELi8ELb0E", "attn_mfma_kernelILi128ELi8ELi8E",
                 "decode_step_kernelILi128ELi4ELb1E", "decode_step_kernelILi128ELi8ELb1E"):
        (name,) = [n for n in res if part in n]
        assert res[name]["waves_per_simd"] == 2, res[name]


def test_noalloc_step_rejects_shapes_beyond_its_static_scratch(L):
    """selective_decode_step_noalloc validates like selective_decode_step and refuses, before any
    HIP call, a shape whose workspace exceeds the static scratch (exact-mass logits of 256
    sequences x 64 heads x 4096 blocks: 256 MiB)."""
    big = shape(B=256, Hq=64, Hkv=1, n=65536, L=16)
    need = L.csa_workspace_size(ctypes.byref(big), csa.CSA_WS_SELECTIVE_DECODE_STEP, 4, 0)
    assert need > csa.CSA_STEP_NOALLOC_SCRATCH_BYTES
    p = FAKE
    rc = L.selective_decode_step_noalloc(ctypes.byref(big), csa.CSA_SCORE_EXACT_MASS, p, p, p, None, None, 4, None,
                                         None, 0, csa.CSA_PROXY_NONE, None, None, p, p, None)
    assert rc == csa.CSA_ERR_WORKSPACE and b"static buffer" in L.csa_last_error()
    s = shape()
    rc = L.selective_decode_step_noalloc(ctypes.byref(s), csa.CSA_SCORE_SUMMARY, p, p, p, p, p, 0, None, None, 0,
                                         csa.CSA_PROXY_NONE, None, None, p, p, None)
    assert rc == csa.CSA_ERR_INVALID_ARG and b"empty virtual-token set" in L.csa_last_error()
    rc = L.selective_decode_step_noalloc(ctypes.byref(s), csa.CSA_SCORE_SUMMARY, p, p, p, None, p, 2, None, None, 0,
                                         csa.CSA_PROXY_COMPLEMENT, None, None, p, p, None)
    assert rc == csa.CSA_ERR_INVALID_ARG and b"Kbar" in L.csa_last_error()


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define CSA_STEP_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == csa.CSA_STEP_NOALLOC_SCRATCH_BYTES


def test_index_checks_toggle(L):
    prev = L.csa_set_index_checks(1)
    try:
        assert L.csa_set_index_checks(0) == 1
        assert L.csa_set_index_checks(0) == 0
    finally:
        L.csa_set_index_checks(prev)


@pytest.mark.parametrize("value", [-1, 2, 7, 99, -(1 << 31), (1 << 31) - 1])
def test_out_of_range_enum_values_are_rejected(L, value):
    """Enum arguments arrive as plain C ints: values outside the enumerators are rejected (the
    host-sanitized build of this file checks that reading them is well defined)."""
    s = shape(dtype=value) if value not in (0, 1) else shape()
    if value not in (0, 1):
        assert sparse(L, s) == csa.CSA_ERR_INVALID_ARG and b"dtype" in L.csa_last_error()
    s = shape()
    if value not in range(0, 6):
        rc = L.block_score(ctypes.byref(s), value, FAKE, FAKE, FAKE, FAKE, 1 << 20, None)
        assert rc == csa.CSA_ERR_INVALID_ARG and b"mode" in L.csa_last_error()
    if value not in (0, 1):
        assert sparse(L, s, proxy=value) == csa.CSA_ERR_INVALID_ARG and b"proxy mode" in L.csa_last_error()
        rc = L.selective_decode_step(ctypes.byref(s), value, FAKE, FAKE, FAKE, FAKE, FAKE, 2, None, None, 0, 1, None,
                                     None, FAKE, FAKE, FAKE, 1 << 20, None)
        assert rc in (csa.CSA_ERR_INVALID_ARG, csa.CSA_ERR_UNSUPPORTED)
    if value not in range(0, 9):
        assert L.csa_workspace_size(ctypes.byref(s), value, 0, 0) == 0 and b"entry" in L.csa_last_error()


def cluster_build(L, s, C=64, r=16, iters=2, ptr=FAKE, U=FAKE, ws=FAKE, wsb=1 << 40):
    p = ptr
    return L.kv_cluster_build(ctypes.byref(s), C, r, iters, p, p, U, p, p, p, p, p, p, p, p, ws, wsb, None)


def test_cluster_build_argument_checks(L):
    s = shape()
    assert cluster_build(L, s, r=5) == csa.CSA_ERR_UNSUPPORTED
    assert cluster_build(L, s, r=64) == csa.CSA_ERR_UNSUPPORTED
    assert cluster_build(L, s, C=8193, r=4) == csa.CSA_ERR_UNSUPPORTED
    assert cluster_build(L, s, C=1024, r=16) == csa.CSA_ERR_UNSUPPORTED  # 1024 x 16 centroids over the LDS
    assert cluster_build(L, s, C=0) == csa.CSA_ERR_INVALID_ARG
    assert cluster_build(L, s, iters=-1) == csa.CSA_ERR_INVALID_ARG
    assert cluster_build(L, s, ptr=None) == csa.CSA_ERR_INVALID_ARG
    assert cluster_build(L, s, U=FAKE + 2) == csa.CSA_ERR_INVALID_ARG
    assert cluster_build(L, s, ws=None, wsb=0) == csa.CSA_ERR_WORKSPACE
    need = csa.workspace_size(s, csa.CSA_WS_KV_CLUSTER_BUILD, 64, 16)
    # projections [B, Hkv, n, r] and centroids [B, Hkv, C, r], fp64
    assert need == ((2 * 2 * 1024 * 16 * 8 + 255) // 256) * 256 + 2 * 2 * 64 * 16 * 8
    assert cluster_build(L, s, wsb=need - 1) == csa.CSA_ERR_WORKSPACE
    assert cluster_build(L, s, ws=FAKE + 16) == csa.CSA_ERR_WORKSPACE  # not 256-byte aligned
    assert csa.workspace_size(s, csa.CSA_WS_KV_CLUSTER_BUILD, 64, 5) == 0


def test_cluster_score_and_attention_argument_checks(L):
    s = shape()
    # G = 4: logits [B, Hq, C] in the workspace
    assert csa.workspace_size(s, csa.CSA_WS_CLUSTER_SCORE, 100, 0) == 2 * 8 * 100 * 4 + 2 * 2 * 4 * 16 * 4
    assert csa.workspace_size(shape(Hq=2), csa.CSA_WS_CLUSTER_SCORE, 100, 0) == 0
    assert L.cluster_score(ctypes.byref(s), 100, FAKE, FAKE, FAKE, FAKE, None, 0, None) == csa.CSA_ERR_WORKSPACE
    assert L.cluster_score(ctypes.byref(s), 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == csa.CSA_ERR_INVALID_ARG
    assert L.cluster_score(ctypes.byref(s), 100, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == \
        csa.CSA_ERR_INVALID_ARG

    def attn(s, C=64, k=4, proxy=csa.CSA_PROXY_COMPLEMENT, sel=FAKE, kc=FAKE):
        return L.cluster_decode_attn(ctypes.byref(s), C, FAKE, FAKE, FAKE, kc, kc, FAKE, sel, k, proxy, FAKE, FAKE,
                                     None)

    assert attn(shape(dtype=csa.CSA_F32)) == csa.CSA_ERR_UNSUPPORTED
    assert attn(shape(Hq=18)) == csa.CSA_ERR_UNSUPPORTED  # G = 9
    assert attn(s, k=65) == csa.CSA_ERR_INVALID_ARG
    assert attn(s, C=1000, k=257) == csa.CSA_ERR_UNSUPPORTED
    assert attn(s, C=9000) == csa.CSA_ERR_UNSUPPORTED
    assert attn(s, k=0, proxy=csa.CSA_PROXY_NONE) == csa.CSA_ERR_INVALID_ARG
    assert attn(s, proxy=2) == csa.CSA_ERR_INVALID_ARG
    assert attn(s, sel=None) == csa.CSA_ERR_INVALID_ARG
    assert attn(s, kc=None) == csa.CSA_ERR_INVALID_ARG


def test_cov_sub_argument_checks(L):
    s = shape()  # d = 128, L = 64
    assert L.kv_cov_sub_build(ctypes.byref(s), 85, None, FAKE, FAKE, None) == csa.CSA_ERR_INVALID_ARG
    assert L.kv_cov_sub_build(ctypes.byref(s), 0, FAKE, FAKE, FAKE, None) == csa.CSA_ERR_INVALID_ARG
    assert L.kv_cov_sub_build(ctypes.byref(s), 129, FAKE, FAKE, FAKE, None) == csa.CSA_ERR_INVALID_ARG
    assert L.kv_cov_sub_build(ctypes.byref(s), 85, FAKE, FAKE + 2, FAKE, None) == csa.CSA_ERR_INVALID_ARG
    big = shape(L=128)
    assert L.kv_cov_sub_build(ctypes.byref(big), 85, FAKE, FAKE, FAKE, None) == csa.CSA_ERR_UNSUPPORTED
    assert csa.cov_sub_block_elems(128, 85) == 128 + 4 * 88
    f32 = shape(dtype=csa.CSA_F32)
    assert L.block_score_cobs2_sub(ctypes.byref(f32), 85, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                                   None) == csa.CSA_ERR_UNSUPPORTED
    assert L.block_score_cobs2_sub(ctypes.byref(shape(Hq=18)), 85, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                                   None) == csa.CSA_ERR_UNSUPPORTED  # G = 9
    assert L.block_score_cobs2_sub(ctypes.byref(s), 85, FAKE, FAKE, FAKE, FAKE, None, 0,
                                   None) == csa.CSA_ERR_WORKSPACE
    assert csa.workspace_size(s, csa.CSA_WS_BLOCK_SCORE_COBS2_SUB) == csa.workspace_size(s, csa.CSA_WS_BLOCK_SCORE_COBS2)


def test_cov_sub4_argument_checks(L):
    s = shape()
    f32 = shape(dtype=csa.CSA_F32)
    assert L.kv_cov_sub4_build(ctypes.byref(f32), 85, FAKE, FAKE, FAKE, None) == csa.CSA_ERR_UNSUPPORTED
    assert L.kv_cov_sub4_build(ctypes.byref(s), 0, FAKE, FAKE, FAKE, None) == csa.CSA_ERR_INVALID_ARG
    assert L.block_score_cobs2_sub4(ctypes.byref(s), 85, FAKE, FAKE, FAKE, FAKE, None, 0,
                                    None) == csa.CSA_ERR_WORKSPACE
    assert csa.cov_sub4_block_bytes(128, 85) == 464 and csa.cov_sub4_block_bytes(64, 30) == 128 + 16 + 4 * 16
