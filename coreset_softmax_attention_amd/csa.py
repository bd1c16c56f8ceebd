"""Thin Python binding of libcsa.so (the C-ABI in include/csa.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch supplies device memory and the current HIP stream.  The same
names as the C entry points are exported.  If the library has not been built,
loading fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

# CSA_LIBRARY names another build of the same library (the host-sanitized build of the tests)
_LIB_PATH = os.environ.get("CSA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")

CSA_OK, CSA_ERR_INVALID_ARG, CSA_ERR_UNSUPPORTED, CSA_ERR_WORKSPACE, CSA_ERR_HIP = 0, -1, -2, -3, -4
CSA_F32, CSA_BF16 = 0, 1
CSA_SCORE_SUMMARY, CSA_SCORE_EXACT_MASS, CSA_SCORE_BOX, CSA_SCORE_COBS2, CSA_SCORE_PROXY_ERROR = 0, 1, 2, 3, 4
CSA_SCORE_COBS2_FP4 = 5
CSA_COBS_RANK = 4
CSA_PROXY_NONE, CSA_PROXY_COMPLEMENT = 0, 1
CSA_WS_BLOCK_SCORE_SUMMARY, CSA_WS_BLOCK_SCORE_EXACT_MASS = 0, 1
CSA_WS_SPARSE_DECODE_ATTN, CSA_WS_DENSE_DECODE_ATTN, CSA_WS_SELECTIVE_DECODE_STEP = 2, 3, 4
CSA_WS_BLOCK_SCORE_BOX, CSA_WS_BLOCK_SCORE_COBS2, CSA_WS_BLOCK_SCORE_PROXY_ERROR = 5, 6, 7
CSA_WS_BLOCK_SCORE_COBS2_FP4 = 8
CSA_WS_KV_CLUSTER_BUILD, CSA_WS_CLUSTER_SCORE, CSA_WS_CLUSTER_DECODE_STEP = 9, 10, 11
CSA_WS_BLOCK_SCORE_COBS2_SUB = 12

MODES = {"summary": CSA_SCORE_SUMMARY, "exact_mass": CSA_SCORE_EXACT_MASS, "box": CSA_SCORE_BOX,
         "cobs2": CSA_SCORE_COBS2, "proxy_error": CSA_SCORE_PROXY_ERROR, "cobs2_fp4": CSA_SCORE_COBS2_FP4}
_SCORE_WS = {"summary": CSA_WS_BLOCK_SCORE_SUMMARY, "exact_mass": CSA_WS_BLOCK_SCORE_EXACT_MASS,
             "box": CSA_WS_BLOCK_SCORE_BOX, "cobs2": CSA_WS_BLOCK_SCORE_COBS2,
             "proxy_error": CSA_WS_BLOCK_SCORE_PROXY_ERROR, "cobs2_fp4": CSA_WS_BLOCK_SCORE_COBS2_FP4}
_SUMMARY_ROWS = {"summary": None, "box": 2, "cobs2": 1 + CSA_COBS_RANK, "proxy_error": 2,
                 "cobs2_fp4": 0}  # rows per block (0: packed bytes)


def cov4_block_bytes(d: int) -> int:
    """Bytes per block of the FP4 second-order descriptor (CSA_COV4_BLOCK_BYTES)."""
    return 2 * d + 4 * CSA_COBS_RANK + CSA_COBS_RANK * d // 2


class CsaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {detail} (status {status})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("n_tokens", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("dtype", ctypes.c_int),
        ("scale", ctypes.c_float),
    ]

    @property
    def n_blocks(self) -> int:
        L = min(self.block_size, self.n_tokens)
        return -(-self.n_tokens // L)


_lib = None
_P, _I32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_SIGS = {
    "kv_summary_build": [ctypes.POINTER(Shape), _P, _P, _P, _P, _P],
    "kv_box_build": [ctypes.POINTER(Shape), _P, _P, _P],
    "kv_cov_build": [ctypes.POINTER(Shape), _P, _P, _P],
    "kv_var_build": [ctypes.POINTER(Shape), _P, _P, _P],
    "kv_cov4_build": [ctypes.POINTER(Shape), _P, _P, _P],
    "block_score": [ctypes.POINTER(Shape), ctypes.c_int, _P, _P, _P, _P, _SZ, _P],
    "topk_select": [_I32, _I32, _I32, _P, _P, _P],
    "sparse_decode_attn": [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _I32, _P, _P, _I32, ctypes.c_int,
                           _P, _P, _P, _SZ, _P],
    "dense_decode_attn": [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _SZ, _P],
    "selective_decode_step": [ctypes.POINTER(Shape), ctypes.c_int, _P, _P, _P, _P, _P, _I32, _P, _P, _I32,
                              ctypes.c_int, _P, _P, _P, _P, _P, _SZ, _P],
    "selective_decode_step_noalloc": [ctypes.POINTER(Shape), ctypes.c_int, _P, _P, _P, _P, _P, _I32, _P, _P, _I32,
                                      ctypes.c_int, _P, _P, _P, _P, _P],
    "kv_cluster_build": [ctypes.POINTER(Shape), _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                         _SZ, _P],
    "cluster_score": [ctypes.POINTER(Shape), _I32, _P, _P, _P, _P, _P, _SZ, _P],
    "cluster_decode_attn": [ctypes.POINTER(Shape), _I32, _P, _P, _P, _P, _P, _P, _P, _I32, ctypes.c_int, _P, _P,
                            _P],
    "kv_cov_sub_build": [ctypes.POINTER(Shape), _I32, _P, _P, _P, _P],
    "block_score_cobs2_sub": [ctypes.POINTER(Shape), _I32, _P, _P, _P, _P, _P, _SZ, _P],
    "kv_cov_sub4_build": [ctypes.POINTER(Shape), _I32, _P, _P, _P, _P],
    "block_score_cobs2_sub4": [ctypes.POINTER(Shape), _I32, _P, _P, _P, _P, _P, _SZ, _P],
    "cluster_decode_step": [ctypes.POINTER(Shape), _I32, _P, _P, _P, _P, _P, _P, _I32, ctypes.c_int, _P, _P, _P, _P,
                            _P, _SZ, _P],
}
CSA_STEP_NOALLOC_SCRATCH_BYTES = 64 << 20


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libcsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m coreset_softmax_attention_amd.build_lib` (or __graft_entry__.build())")
        L = ctypes.CDLL(_LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.csa_workspace_size.argtypes = [ctypes.POINTER(Shape), ctypes.c_int, _I32, _I32]
        L.csa_workspace_size.restype = _SZ
        L.csa_status_str.argtypes = [ctypes.c_int]
        L.csa_status_str.restype = ctypes.c_char_p
        L.csa_last_error.argtypes = []
        L.csa_last_error.restype = ctypes.c_char_p
        L.csa_set_index_checks.argtypes = [ctypes.c_int]
        L.csa_set_index_checks.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, where: str):
    if rc != CSA_OK:
        raise CsaError(rc, where, lib().csa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")
    return ts[0].device


def make_shape(q: torch.Tensor, K: torch.Tensor, block_size: int, scale: float = 0.0) -> Shape:
    """Shape of q [B, Hq, d] against a cache K [B, Hkv, n, d]."""
    B, Hq, d = q.shape
    B2, Hkv, n, d2 = K.shape
    if B != B2 or d != d2:
        raise ValueError(f"q {tuple(q.shape)} does not match K {tuple(K.shape)}")
    if q.dtype != K.dtype:
        raise TypeError("q and K must have the same dtype")
    return Shape(B, Hq, Hkv, d, n, block_size, _dtype_code(K), float(scale))


def workspace_size(shape: Shape, entry: int, k: int = 0, m: int = 0) -> int:
    return int(lib().csa_workspace_size(ctypes.byref(shape), entry, k, m))


def _workspace(shape: Shape, entry: int, k: int, m: int, ws, device):
    need = workspace_size(shape, entry, k, m)
    if need == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def kv_summary_build(K: torch.Tensor, V: torch.Tensor, block_size: int, Kbar=None, Vbar=None):
    """Mean key and mean value of every block: Kbar, Vbar [B, Hkv, nb, d]."""
    dev = _dev(K, V, Kbar, Vbar)
    B, Hkv, n, d = K.shape
    shape = Shape(B, Hkv, Hkv, d, n, block_size, _dtype_code(K), 0.0)
    nb = shape.n_blocks
    Kbar = torch.empty((B, Hkv, nb, d), dtype=K.dtype, device=dev) if Kbar is None else Kbar
    Vbar = torch.empty((B, Hkv, nb, d), dtype=K.dtype, device=dev) if Vbar is None else Vbar
    _check(lib().kv_summary_build(ctypes.byref(shape), _ptr(K), _ptr(V), _ptr(Kbar), _ptr(Vbar), _stream(dev)),
           "kv_summary_build")
    return Kbar, Vbar


def kv_box_build(K: torch.Tensor, block_size: int, Kbox=None):
    """Element-wise minimum and maximum key of every block: Kbox [B, Hkv, nb, 2, d]."""
    dev = _dev(K, Kbox)
    B, Hkv, n, d = K.shape
    shape = Shape(B, Hkv, Hkv, d, n, block_size, _dtype_code(K), 0.0)
    Kbox = torch.empty((B, Hkv, shape.n_blocks, 2, d), dtype=K.dtype, device=dev) if Kbox is None else Kbox
    _check(lib().kv_box_build(ctypes.byref(shape), _ptr(K), _ptr(Kbox), _stream(dev)), "kv_box_build")
    return Kbox


def kv_cov_build(K: torch.Tensor, block_size: int, Kcov=None):
    """Second-order descriptors: Kcov [B, Hkv, nb, 1 + CSA_COBS_RANK, d] (mean key, then the
    top scaled eigenvectors of each block's key covariance)."""
    dev = _dev(K, Kcov)
    B, Hkv, n, d = K.shape
    shape = Shape(B, Hkv, Hkv, d, n, block_size, _dtype_code(K), 0.0)
    if Kcov is None:
        Kcov = torch.empty((B, Hkv, shape.n_blocks, 1 + CSA_COBS_RANK, d), dtype=K.dtype, device=dev)
    _check(lib().kv_cov_build(ctypes.byref(shape), _ptr(K), _ptr(Kcov), _stream(dev)), "kv_cov_build")
    return Kcov


def kv_cov4_build(K: torch.Tensor, block_size: int, Kcov4=None):
    """Second-order descriptors with FP4 (E2M1) eigenvectors: Kcov4 uint8
    [B, Hkv, nb, cov4_block_bytes(d)] (bfloat16 mean key, fp32 scales, 4-bit codes)."""
    dev = _dev(K, Kcov4)
    B, Hkv, n, d = K.shape
    shape = Shape(B, Hkv, Hkv, d, n, block_size, _dtype_code(K), 0.0)
    if Kcov4 is None:
        Kcov4 = torch.empty((B, Hkv, shape.n_blocks, cov4_block_bytes(d)), dtype=torch.uint8, device=dev)
    _check(lib().kv_cov4_build(ctypes.byref(shape), _ptr(K), _ptr(Kcov4), _stream(dev)), "kv_cov4_build")
    return Kcov4


def cov_sub_block_elems(d: int, s_dim: int) -> int:
    """Elements per block of the query-subspace descriptor (CSA_COV_SUB_BLOCK_ELEMS)."""
    return d + CSA_COBS_RANK * (-(-s_dim // 8) * 8)


def cov_sub4_block_bytes(d: int, s_dim: int) -> int:
    """Bytes per block of the FP4 query-subspace descriptor (CSA_COV_SUB4_BLOCK_BYTES)."""
    return 2 * d + 4 * CSA_COBS_RANK + CSA_COBS_RANK * (-(-s_dim // 32) * 32) // 2


def kv_cov_sub_build(K: torch.Tensor, U: torch.Tensor, block_size: int, Kcs=None, fp4: bool = False):
    """Query-subspace second-order descriptors from the basis U [Hkv, d, s] (float32):
    [B, Hkv, nb, cov_sub_block_elems(d, s)] in the cache dtype, or with fp4
    [B, Hkv, nb, cov_sub4_block_bytes(d, s)] bytes."""
    dev = _dev(K, U, Kcs)
    B, Hkv, n, d = K.shape
    s_dim = U.shape[-1]
    shape = Shape(B, Hkv, Hkv, d, n, block_size, _dtype_code(K), 0.0)
    nb = shape.n_blocks
    if Kcs is None:
        Kcs = (torch.empty((B, Hkv, nb, cov_sub4_block_bytes(d, s_dim)), dtype=torch.uint8, device=dev) if fp4 else
               torch.empty((B, Hkv, nb, cov_sub_block_elems(d, s_dim)), dtype=K.dtype, device=dev))
    name = "kv_cov_sub4_build" if fp4 else "kv_cov_sub_build"
    _check(getattr(lib(), name)(ctypes.byref(shape), s_dim, _ptr(K), _ptr(U), _ptr(Kcs), _stream(dev)), name)
    return Kcs


def block_score_cobs2_sub(q: torch.Tensor, Kcs: torch.Tensor, U: torch.Tensor, block_size: int, n_tokens: int,
                          scale: float = 0.0, scores=None, ws=None, fp4: bool = False):
    """Second-order block scores [B, Hkv, nb] from query-subspace descriptors (FP4 ones with fp4)."""
    dev = _dev(q, Kcs, U)
    B, Hq, d = q.shape
    Hkv, nb = Kcs.shape[1], Kcs.shape[2]
    s_dim = U.shape[-1]
    shape = Shape(B, Hq, Hkv, d, n_tokens, block_size, _dtype_code(q), float(scale))
    scores = torch.empty((B, Hkv, nb), dtype=torch.float32, device=dev) if scores is None else scores
    ws, wsb = _workspace(shape, CSA_WS_BLOCK_SCORE_COBS2_SUB, 0, 0, ws, dev)
    name = "block_score_cobs2_sub4" if fp4 else "block_score_cobs2_sub"
    _check(getattr(lib(), name)(ctypes.byref(shape), s_dim, _ptr(q), _ptr(Kcs), _ptr(U), _ptr(scores), _ptr(ws), wsb,
                                _stream(dev)), name)
    return scores


def kv_var_build(K: torch.Tensor, block_size: int, Kvar=None):
    """Mean and variance tokens of every block: Kvar [B, Hkv, nb, 2, d] (row 0 the mean key,
    row 1 the per-coordinate key variance), for the proxy-error scores."""
    dev = _dev(K, Kvar)
    B, Hkv, n, d = K.shape
    shape = Shape(B, Hkv, Hkv, d, n, block_size, _dtype_code(K), 0.0)
    Kvar = torch.empty((B, Hkv, shape.n_blocks, 2, d), dtype=K.dtype, device=dev) if Kvar is None else Kvar
    _check(lib().kv_var_build(ctypes.byref(shape), _ptr(K), _ptr(Kvar), _stream(dev)), "kv_var_build")
    return Kvar


def block_score(q: torch.Tensor, keys: torch.Tensor, mode: str, block_size: int, n_tokens: int | None = None,
                scale: float = 0.0, scores=None, ws=None):
    """Block scores [B, Hkv, nb].  keys = Kbar (mode 'summary'), K (mode 'exact_mass'), Kbox
    (mode 'box'), Kcov (mode 'cobs2') or Kvar (mode 'proxy_error'); n_tokens is needed in every mode but 'exact_mass' (the
    cache length the summaries describe)."""
    dev = _dev(q, keys, scores)
    B, Hq, d = q.shape
    Hkv = keys.shape[1]
    if mode in _SUMMARY_ROWS:
        if n_tokens is None:
            raise ValueError(f"{mode} mode needs n_tokens")
        n = n_tokens
    else:
        n = keys.shape[2]
    shape = Shape(B, Hq, Hkv, d, n, block_size, _dtype_code(q), float(scale))
    nb = shape.n_blocks
    if mode in _SUMMARY_ROWS and keys.shape[2] != nb:
        raise ValueError(f"the summaries have {keys.shape[2]} blocks, expected {nb}")
    rows = _SUMMARY_ROWS.get(mode)
    if rows == 0:
        if keys.dim() != 4 or keys.dtype != torch.uint8 or keys.shape[3] != cov4_block_bytes(d):
            raise ValueError(f"{mode} mode needs keys uint8 [B, Hkv, nb, {cov4_block_bytes(d)}]")
    elif rows is not None and (keys.dim() != 5 or keys.shape[3] != rows):
        raise ValueError(f"{mode} mode needs keys [B, Hkv, nb, {rows}, d]")
    scores = torch.empty((B, Hkv, nb), dtype=torch.float32, device=dev) if scores is None else scores
    ws, wsb = _workspace(shape, _SCORE_WS[mode], 0, 0, ws, dev)
    _check(lib().block_score(ctypes.byref(shape), MODES[mode], _ptr(q), _ptr(keys), _ptr(scores), _ptr(ws), wsb,
                             _stream(dev)), "block_score")
    return scores


def topk_select(scores: torch.Tensor, k: int, sel=None):
    """Top-k block indices per row (ascending), ties to the lower index: [..., min(k, nb)] int32."""
    dev = _dev(scores, sel)
    nb = scores.shape[-1]
    rows = scores.numel() // nb
    kk = min(k, nb)
    sel = torch.empty(scores.shape[:-1] + (kk,), dtype=torch.int32, device=dev) if sel is None else sel
    _check(lib().topk_select(rows, nb, k, _ptr(scores), _ptr(sel), _stream(dev)), "topk_select")
    return sel


def sparse_decode_attn(q, K, V, Kbar, Vbar, sel, block_size: int, proxies: bool = True, tok_idx=None,
                       tok_logw=None, scale: float = 0.0, out=None, lse=None, ws=None):
    """Attention over exact tokens of sel, optional weighted tokens and count-aware proxies.
    Returns (out [B, Hq, d] float32, lse [B, Hq] float32)."""
    dev = _dev(q, K, V, Kbar, Vbar, sel, tok_idx, tok_logw)
    shape = make_shape(q, K, block_size, scale)
    k = sel.shape[-1] if sel is not None else 0
    m = tok_idx.shape[-1] if tok_idx is not None else 0
    B, Hq, d = q.shape
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    ws, wsb = _workspace(shape, CSA_WS_SPARSE_DECODE_ATTN, k, m, ws, dev)
    _check(lib().sparse_decode_attn(ctypes.byref(shape), _ptr(q), _ptr(K), _ptr(V), _ptr(Kbar), _ptr(Vbar),
                                    _ptr(sel), k, _ptr(tok_idx), _ptr(tok_logw), m,
                                    CSA_PROXY_COMPLEMENT if proxies else CSA_PROXY_NONE, _ptr(out), _ptr(lse),
                                    _ptr(ws), wsb, _stream(dev)), "sparse_decode_attn")
    return out, lse


def dense_decode_attn(q, K, V, scale: float = 0.0, out=None, lse=None, ws=None):
    """Softmax attention over every token: (out [B, Hq, d], lse [B, Hq])."""
    dev = _dev(q, K, V)
    shape = make_shape(q, K, K.shape[2], scale)
    B, Hq, d = q.shape
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    ws, wsb = _workspace(shape, CSA_WS_DENSE_DECODE_ATTN, 0, 0, ws, dev)
    _check(lib().dense_decode_attn(ctypes.byref(shape), _ptr(q), _ptr(K), _ptr(V), _ptr(out), _ptr(lse), _ptr(ws),
                                   wsb, _stream(dev)), "dense_decode_attn")
    return out, lse


def selective_decode_step(q, K, V, Kbar, Vbar, k: int, block_size: int, mode: str = "summary",
                          proxies: bool = True, tok_idx=None, tok_logw=None, scale: float = 0.0, scores=None,
                          sel=None, out=None, lse=None, ws=None, want_scores: bool = False, want_sel: bool = False):
    """block_score -> topk_select -> sparse_decode_attn in one call (one kernel where the shape
    allows).  Returns (out, lse, scores or None, sel or None)."""
    dev = _dev(q, K, V, Kbar, Vbar, tok_idx, tok_logw)
    shape = make_shape(q, K, block_size, scale)
    m = tok_idx.shape[-1] if tok_idx is not None else 0
    B, Hq, d = q.shape
    Hkv, nb = K.shape[1], shape.n_blocks
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    if want_scores and scores is None:
        scores = torch.empty((B, Hkv, nb), dtype=torch.float32, device=dev)
    if want_sel and sel is None:
        sel = torch.empty((B, Hkv, min(k, nb)), dtype=torch.int32, device=dev)
    ws, wsb = _workspace(shape, CSA_WS_SELECTIVE_DECODE_STEP, k, m, ws, dev)
    _check(lib().selective_decode_step(ctypes.byref(shape), MODES[mode], _ptr(q), _ptr(K), _ptr(V), _ptr(Kbar),
                                       _ptr(Vbar), k, _ptr(tok_idx), _ptr(tok_logw), m,
                                       CSA_PROXY_COMPLEMENT if proxies else CSA_PROXY_NONE, _ptr(scores),
                                       _ptr(sel), _ptr(out), _ptr(lse), _ptr(ws), wsb, _stream(dev)),
           "selective_decode_step")
    return out, lse, scores, sel


def selective_decode_step_noalloc(q, K, V, Kbar, Vbar, k: int, block_size: int, mode: str = "summary",
                                  proxies: bool = True, tok_idx=None, tok_logw=None, scale: float = 0.0,
                                  scores=None, sel=None, out=None, lse=None):
    """selective_decode_step without a workspace: the library's static per-GPU scratch serves
    instead (calls overlapping on one GPU race).  All outputs must be given (nothing is
    allocated here either, so the call can sit inside a capture that forbids allocation);
    scores and sel may be None.  Returns (out, lse, scores, sel)."""
    dev = _dev(q, K, V, Kbar, Vbar, tok_idx, tok_logw)
    if out is None or lse is None:
        raise ValueError("selective_decode_step_noalloc: out and lse must be given")
    shape = make_shape(q, K, block_size, scale)
    m = tok_idx.shape[-1] if tok_idx is not None else 0
    _check(lib().selective_decode_step_noalloc(ctypes.byref(shape), MODES[mode], _ptr(q), _ptr(K), _ptr(V),
                                               _ptr(Kbar), _ptr(Vbar), k, _ptr(tok_idx), _ptr(tok_logw), m,
                                               CSA_PROXY_COMPLEMENT if proxies else CSA_PROXY_NONE, _ptr(scores),
                                               _ptr(sel), _ptr(out), _ptr(lse), _stream(dev)),
           "selective_decode_step_noalloc")
    return out, lse, scores, sel


def kv_cluster_build(K: torch.Tensor, V: torch.Tensor, U: torch.Tensor, seeds: torch.Tensor, iters: int,
                     out: dict | None = None, ws=None) -> dict:
    """Query-guided clusters of each KV head's keys: k-means of K U (U [B, Hkv, d, r] float32)
    from the seed tokens seeds [B, Hkv, C] (int32), `iters` rounds and a final assignment.
    Returns a dict of assign, order [B, Hkv, n], offsets [B, Hkv, C + 1] (int32), Kg, Vg
    [B, Hkv, n, d] (the cache in cluster order) and Kc, Vc [B, Hkv, C, d] (cluster means);
    tensors given in `out` are written in place."""
    dev = _dev(K, V, U, seeds)
    B, Hkv, n, d = K.shape
    C, r = seeds.shape[-1], U.shape[-1]
    shape = Shape(B, Hkv, Hkv, d, n, n, _dtype_code(K), 0.0)
    o = dict(out or {})
    want = {"assign": ((B, Hkv, n), torch.int32), "order": ((B, Hkv, n), torch.int32),
            "offsets": ((B, Hkv, C + 1), torch.int32), "Kg": ((B, Hkv, n, d), K.dtype),
            "Vg": ((B, Hkv, n, d), K.dtype), "Kc": ((B, Hkv, C, d), K.dtype), "Vc": ((B, Hkv, C, d), K.dtype)}
    for name, (shp, dt) in want.items():
        if o.get(name) is None:
            o[name] = torch.empty(shp, dtype=dt, device=dev)
    ws, wsb = _workspace(shape, CSA_WS_KV_CLUSTER_BUILD, C, r, ws, dev)
    _check(lib().kv_cluster_build(ctypes.byref(shape), C, r, iters, _ptr(K), _ptr(V), _ptr(U), _ptr(seeds),
                                  _ptr(o["assign"]), _ptr(o["order"]), _ptr(o["offsets"]), _ptr(o["Kg"]),
                                  _ptr(o["Vg"]), _ptr(o["Kc"]), _ptr(o["Vc"]), _ptr(ws), wsb, _stream(dev)),
           "kv_cluster_build")
    return o


def cluster_score(q: torch.Tensor, Kc: torch.Tensor, offsets: torch.Tensor, n_tokens: int, scale: float = 0.0,
                  scores=None, ws=None):
    """Cluster scores [B, Hkv, C]: scale q.Kc + ln count per head, combined by the block-score group rule."""
    dev = _dev(q, Kc, offsets)
    B, Hq, d = q.shape
    _, Hkv, C, _ = Kc.shape
    shape = Shape(B, Hq, Hkv, d, n_tokens, n_tokens, _dtype_code(Kc), float(scale))
    scores = torch.empty((B, Hkv, C), dtype=torch.float32, device=dev) if scores is None else scores
    ws, wsb = _workspace(shape, CSA_WS_CLUSTER_SCORE, C, 0, ws, dev)
    _check(lib().cluster_score(ctypes.byref(shape), C, _ptr(q), _ptr(Kc), _ptr(offsets), _ptr(scores), _ptr(ws), wsb,
                               _stream(dev)), "cluster_score")
    return scores


def cluster_decode_attn(q, Kg, Vg, Kc, Vc, offsets, sel, proxies: bool = True, scale: float = 0.0, out=None,
                        lse=None):
    """Attention over every token of the selected clusters (rows of Kg, Vg) and one proxy per
    other non-empty cluster.  Returns (out [B, Hq, d] float32, lse [B, Hq] float32)."""
    dev = _dev(q, Kg, Vg, Kc, Vc, offsets, sel)
    shape = make_shape(q, Kg, Kg.shape[2], scale)
    C = offsets.shape[-1] - 1
    k = sel.shape[-1] if sel is not None else 0
    B, Hq, d = q.shape
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    _check(lib().cluster_decode_attn(ctypes.byref(shape), C, _ptr(q), _ptr(Kg), _ptr(Vg), _ptr(Kc), _ptr(Vc),
                                     _ptr(offsets), _ptr(sel), k,
                                     CSA_PROXY_COMPLEMENT if proxies else CSA_PROXY_NONE, _ptr(out), _ptr(lse),
                                     _stream(dev)), "cluster_decode_attn")
    return out, lse


def cluster_decode_step(q, Kg, Vg, Kc, Vc, offsets, k: int, proxies: bool = True, scale: float = 0.0, scores=None,
                        sel=None, out=None, lse=None, ws=None, want_scores: bool = False, want_sel: bool = False):
    """cluster_score -> topk_select -> cluster_decode_attn in one call.
    Returns (out, lse, scores or None, sel or None)."""
    dev = _dev(q, Kg, Vg, Kc, Vc, offsets)
    shape = make_shape(q, Kg, Kg.shape[2], scale)
    C = offsets.shape[-1] - 1
    B, Hq, d = q.shape
    Hkv = Kg.shape[1]
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    if want_scores and scores is None:
        scores = torch.empty((B, Hkv, C), dtype=torch.float32, device=dev)
    if want_sel and sel is None:
        sel = torch.empty((B, Hkv, min(k, C)), dtype=torch.int32, device=dev)
    ws, wsb = _workspace(shape, CSA_WS_CLUSTER_DECODE_STEP, k, C, ws, dev)
    _check(lib().cluster_decode_step(ctypes.byref(shape), C, _ptr(q), _ptr(Kg), _ptr(Vg), _ptr(Kc), _ptr(Vc),
                                     _ptr(offsets), k, CSA_PROXY_COMPLEMENT if proxies else CSA_PROXY_NONE,
                                     _ptr(scores), _ptr(sel), _ptr(out), _ptr(lse), _ptr(ws), wsb, _stream(dev)),
           "cluster_decode_step")
    return out, lse, scores, sel


def set_index_checks(enable: bool) -> bool:
    """Turn the host-side check of device-resident index arrays on or off (csa_set_index_checks);
    returns the previous setting."""
    return bool(lib().csa_set_index_checks(1 if enable else 0))


def to_device(a, device="cuda"):
    """numpy array from the workload generator -> torch tensor on the GPU
    (uint16 bfloat16 patterns become torch.bfloat16)."""
    import numpy as np

    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)
