"""NumPy front end of the fp64 CPU oracle (csa_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg of
the benchmark may import this module; the product path never does.  It shares no
code with the HIP library and imports nothing from it.

Arrays follow the layouts in csa_oracle.h.  Stored tensors are numpy arrays of
dtype float32 (binary32) or uint16 (bfloat16 bit patterns); every result is fp64.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libcsa_oracle.so")

SUMMARY, EXACT_MASS, BOX, COBS2, PROXY_ERROR, COBS2_FP4 = 0, 1, 2, 3, 4, 5
COBS_RANK = 4  # scaled eigenvectors per block in the second-order descriptor


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, no FMA contraction, OpenMP over pairs)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
             _SRC, "-o", tmp, "-lm"],
            cwd=_HERE,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int),
        ("n_q_heads", ctypes.c_int),
        ("n_kv_heads", ctypes.c_int),
        ("head_dim", ctypes.c_int),
        ("n_tokens", ctypes.c_int),
        ("block_size", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("scale", ctypes.c_double),
    ]


@dataclass(frozen=True)
class Shape:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_tokens: int
    block_size: int
    dtype: str  # "f32" or "bf16"
    scale: float = 0.0  # 0 means 1/sqrt(head_dim)

    @property
    def n_blocks(self) -> int:
        return -(-self.n_tokens // self.block_size)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def c(self) -> _Shape:
        return _Shape(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim, self.n_tokens,
                      self.block_size, 0 if self.dtype == "f32" else 1, float(self.scale))

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == "f32" else np.uint16


_lib = None
_lib_override = None


def use_library(path):
    """Load the oracle from another build of csa_oracle.c (None restores the default).
    Used by the mutation tests, which build copies with planted mistakes."""
    global _lib, _lib_override
    _lib, _lib_override = None, path


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(_lib_override or build())
        P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_double)
        SP = ctypes.POINTER(_Shape)
        lib.oracle_kv_summary_build.argtypes = [SP, P, P, P, P]
        lib.oracle_block_logits.argtypes = [SP, I, P, P, P]
        lib.oracle_group_score.argtypes = [SP, P, P]
        lib.oracle_topk.argtypes = [I, I, I, P, P, P]
        lib.oracle_attend.argtypes = [SP, P, P, P, P, P, P, I, P, P, I, I, P, P]
        lib.oracle_dense.argtypes = [SP, P, P, P, P, P]
        lib.oracle_block_mass.argtypes = [SP, P, P, P, P, P]
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_bf16.restype = ctypes.c_uint16
        lib.oracle_kv_box_build.argtypes = [SP, P, P]
        lib.oracle_kv_box_build.restype = I
        lib.oracle_store_array.argtypes = [I, ctypes.c_size_t, P, P]
        lib.oracle_store_array.restype = I
        lib.oracle_cluster_build.argtypes = [SP, I, I, I, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_cluster_build.restype = I
        lib.oracle_cluster_logits.argtypes = [SP, I, P, P, P, P]
        lib.oracle_cluster_logits.restype = I
        lib.oracle_cluster_attend.argtypes = [SP, I, P, P, P, P, P, P, P, P, I, I, P, P]
        lib.oracle_cluster_attend.restype = I
        for f in ("oracle_kv_summary_build", "oracle_block_logits", "oracle_group_score",
                  "oracle_topk", "oracle_attend", "oracle_dense", "oracle_block_mass"):
            getattr(lib, f).restype = I
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _stored(shape: Shape, a, dims):
    a = np.ascontiguousarray(a)
    if a.dtype != shape.np_dtype:
        raise TypeError(f"expected {shape.np_dtype} array, got {a.dtype}")
    if tuple(a.shape) != tuple(dims):
        raise ValueError(f"expected shape {dims}, got {a.shape}")
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid argument")


def kv_summary_build(shape: Shape, K, V):
    """Mean key and mean value of every block, rounded once to the storage dtype."""
    kv = (shape.batch, shape.n_kv_heads, shape.n_tokens, shape.head_dim)
    sm = (shape.batch, shape.n_kv_heads, shape.n_blocks, shape.head_dim)
    K, V = _stored(shape, K, kv), _stored(shape, V, kv)
    Kbar = np.empty(sm, shape.np_dtype)
    Vbar = np.empty(sm, shape.np_dtype)
    _check(_load().oracle_kv_summary_build(ctypes.byref(shape.c()), _ptr(K), _ptr(V), _ptr(Kbar), _ptr(Vbar)),
           "kv_summary_build")
    return Kbar, Vbar


def kv_box_build(shape: Shape, K):
    """Element-wise minimum and maximum key of every block, [B, Hkv, nb, 2, d]."""
    kv = (shape.batch, shape.n_kv_heads, shape.n_tokens, shape.head_dim)
    K = _stored(shape, K, kv)
    Kbox = np.empty((shape.batch, shape.n_kv_heads, shape.n_blocks, 2, shape.head_dim), shape.np_dtype)
    _check(_load().oracle_kv_box_build(ctypes.byref(shape.c()), _ptr(K), _ptr(Kbox)), "kv_box_build")
    return Kbox


def store_array(shape_or_dtype, x):
    """fp64 array -> stored array (binary32, or bfloat16 bit patterns), rounded once."""
    dt = shape_or_dtype.dtype if isinstance(shape_or_dtype, Shape) else shape_or_dtype
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty(x.shape, np.float32 if dt == "f32" else np.uint16)
    _check(_load().oracle_store_array(0 if dt == "f32" else 1, x.size, _ptr(x), _ptr(out)), "store_array")
    return out


def cov_build(shape: Shape, K, Kbar=None, rank: int = COBS_RANK):
    """Second-order block descriptors of "COBS: Cumulant Order Block Sparse Attention": per
    block the mean key and the top-`rank` scaled eigenvectors xi_i = sqrt(lambda_i) u_i of the
    within-block key covariance Sigma_b = (1/c) sum_i (k_i - kbar)(k_i - kbar)^T (the second
    cumulant of the block's keys; the low-rank spectral form of the section on compressing the
    covariance).  Returns [B, Hkv, nb, 1 + rank, d] in the storage dtype: row 0 the mean key
    (the same bits as kv_summary_build), rows 1.. the eigenvectors by decreasing eigenvalue,
    each signed so that its largest-magnitude coordinate is positive."""
    B, Hkv, n, d, L, nb = shape.batch, shape.n_kv_heads, shape.n_tokens, shape.head_dim, shape.block_size, \
        shape.n_blocks
    Kf = widen(shape, _stored(shape, K, (B, Hkv, n, d)))
    if Kbar is None:
        Kbar, _ = kv_summary_build(shape, K, K)
    xi = np.zeros((B, Hkv, nb, rank, d), np.float64)
    for b in range(B):
        for j in range(Hkv):
            for blk in range(nb):
                X = Kf[b, j, blk * L:min(n, (blk + 1) * L)]
                Xc = X - X.mean(axis=0)
                lam, U = np.linalg.eigh(Xc.T @ Xc / X.shape[0])  # ascending
                for i in range(min(rank, d)):
                    u = U[:, d - 1 - i]
                    u = u if u[np.argmax(np.abs(u))] > 0 else -u
                    xi[b, j, blk, i] = math.sqrt(max(lam[d - 1 - i], 0.0)) * u
    out = np.empty((B, Hkv, nb, 1 + rank, d), shape.np_dtype)
    out[:, :, :, 0] = np.asarray(Kbar).reshape(B, Hkv, nb, d)
    out[:, :, :, 1:] = store_array(shape, xi)
    return out


def cobs2_logits(shape: Shape, q, Kcov):
    """Second-order block logits [B, Hq, nb] ([COBS] cumulant expansion truncated at second
    order, with the rank-r covariance): scale q.kbar_b + ln c_b + (1/2) scale^2 sum_i (q.xi_i)^2,
    from the stored descriptors."""
    B, Hq, Hkv, d, nb = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.n_blocks
    G = Hq // Hkv
    qf = widen(shape, _stored(shape, q, (B, Hq, d)))
    C = widen(shape, np.asarray(Kcov)).reshape(B, Hkv, nb, -1, d)
    scale = shape.scale if shape.scale else 1.0 / math.sqrt(d)
    counts = np.array([min(shape.block_size, shape.n_tokens - i * shape.block_size) for i in range(nb)], np.float64)
    out = np.empty((B, Hq, nb), np.float64)
    for h in range(Hq):
        dots = np.einsum("bd,bkrd->bkr", qf[:, h], C[:, h // G])  # [B, nb, 1 + r]
        out[:, h] = scale * dots[:, :, 0] + np.log(counts) + 0.5 * scale * scale * (dots[:, :, 1:] ** 2).sum(-1)
    return out


def var_build(shape: Shape, K, Kbar=None):
    """Mean and variance tokens of every block, the cached pair that the proxy-error ranking of
    "OpenAttention reads 1% of the KV cache -- Count-aware tail proxy" reads (section "Three
    helpers that make the proxy accurate").  Returns [B, Hkv, nb, 2, d] in the storage dtype:
    row 0 the mean key (the bits of kv_summary_build), row 1 the per-coordinate population
    variance of the block's keys about their exact mean, (1/c) sum_i (k_i - mean)^2.  Both
    sums run token by token in fp64; the variance is rounded once."""
    B, Hkv, n, d, L, nb = shape.batch, shape.n_kv_heads, shape.n_tokens, shape.head_dim, shape.block_size, \
        shape.n_blocks
    Kf = widen(shape, _stored(shape, K, (B, Hkv, n, d)))
    if Kbar is None:
        Kbar, _ = kv_summary_build(shape, K, K)
    var = np.empty((B, Hkv, nb, d), np.float64)
    for blk in range(nb):
        X = Kf[:, :, blk * L:min(n, (blk + 1) * L)]  # [B, Hkv, c, d]
        c = X.shape[2]
        s1 = np.zeros((B, Hkv, d))
        for i in range(c):
            s1 = s1 + X[:, :, i]
        mean = s1 / c
        s2 = np.zeros((B, Hkv, d))
        for i in range(c):
            dv = X[:, :, i] - mean
            s2 = s2 + dv * dv
        var[:, :, blk] = s2 / c
    out = np.empty((B, Hkv, nb, 2, d), shape.np_dtype)
    out[:, :, :, 0] = np.asarray(Kbar).reshape(B, Hkv, nb, d)
    out[:, :, :, 1] = store_array(shape, var)
    return out


def proxy_error_logits(shape: Shape, q, Kvar):
    """Per query head h and block b, from the stored mean and variance tokens:
    shat_hb = scale q_h.kbar_b + ln c_b, the log-mass of the block's count-aware proxy
    ("OpenAttention ... Count-aware tail proxy", section "Skipping reviews without losing the
    verdict": mean logit plus ln count), and the log of the proxy's estimated weight error,
    read as the proxy mass times the standard deviation of its block's logits (same section),
    shat_hb + ln sigma_hb with
    sigma_hb = scale sqrt(sum_t q_ht^2 var_bt), the standard deviation of the block's logits
    when its key coordinates are uncorrelated (-inf when sigma = 0).  Returns (shat, lerr),
    each [B, Hq, nb]."""
    B, Hq, Hkv, d, nb = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.n_blocks
    G = Hq // Hkv
    qf = widen(shape, _stored(shape, q, (B, Hq, d)))
    C = widen(shape, np.asarray(Kvar)).reshape(B, Hkv, nb, 2, d)
    scale = shape.scale if shape.scale else 1.0 / math.sqrt(d)
    counts = np.array([min(shape.block_size, shape.n_tokens - i * shape.block_size) for i in range(nb)], np.float64)
    shat = np.empty((B, Hq, nb))
    lerr = np.empty((B, Hq, nb))
    for h in range(Hq):
        mean_dot = np.einsum("bd,bkd->bk", qf[:, h], C[:, h // G, :, 0])
        spread2 = scale * scale * np.einsum("bd,bkd->bk", qf[:, h] ** 2, C[:, h // G, :, 1])
        shat[:, h] = scale * mean_dot + np.log(counts)
        with np.errstate(divide="ignore"):
            lerr[:, h] = np.where(spread2 > 0, shat[:, h] + 0.5 * np.log(np.where(spread2 > 0, spread2, 1.0)),
                                  -np.inf)
    return shat, lerr


def _lse(x, axis):
    m = np.max(x, axis=axis, keepdims=True)
    mf = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        return np.squeeze(mf + np.log(np.sum(np.exp(x - mf), axis=axis, keepdims=True)), axis)


def proxy_error_score(shape: Shape, q, Kvar):
    """Block scores [B, Hkv, nb] of the proxy-error ranking: exact reads go to the blocks whose
    proxies would leave the largest weight error ("OpenAttention ... Count-aware tail proxy",
    section "Three helpers that make the proxy accurate").  G = 1: the log-error itself.  G > 1:
    ln sum_h exp(lerr_hb - ln sum_b' exp(shat_hb')), each head's error as a share of its
    proxy-estimated softmax denominator, added over the group as in the additive GQA score of
    "COBS: Cumulant Order Block Sparse Attention", Eq. (5)."""
    B, Hq, Hkv, nb = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.n_blocks
    G = Hq // Hkv
    shat, lerr = proxy_error_logits(shape, q, Kvar)
    if G == 1:
        return lerr.reshape(B, Hkv, nb)
    rel = lerr - _lse(shat, axis=2)[:, :, None]  # [B, Hq, nb]
    return _lse(rel.reshape(B, Hkv, G, nb), axis=2)


# E2M1 (FP4) magnitudes by 3-bit code: exponent bits 2-1, mantissa bit 0.
E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def fp4_block_bytes(d: int, rank: int = COBS_RANK) -> int:
    """Bytes per block of the FP4 second-order descriptor: the bfloat16 mean key, one fp32
    scale per eigenvector, then the eigenvectors' 4-bit codes (two per byte)."""
    return 2 * d + 4 * rank + rank * d // 2


def e2m1_code(r: np.float32) -> int:
    """4-bit E2M1 code of r (binary32) rounded to the nearest grid value, ties to the even
    mantissa (code bit 0 clear); zero magnitudes are +0."""
    a = abs(float(r))
    best = 0
    for c in range(1, 8):
        d_new, d_old = abs(a - E2M1[c]), abs(a - E2M1[best])
        if d_new < d_old or (d_new == d_old and c % 2 == 0 and best % 2 == 1):
            best = c
    return best | (8 if (float(r) < 0 and best) else 0)


def cov4_pack(shape: Shape, Kcov):
    """FP4 storage of the second-order descriptors ("COBS: Cumulant Order Block Sparse
    Attention", section on quantising the stored factors: E2M1 codes, one fp32 scale per
    eigenvector, the block mean in bfloat16), from the stored bfloat16 descriptors Kcov
    [B, Hkv, nb, 1 + r, d].  Per block: the mean row (its bits), the scales
    s_i = max_t |xi_it| / 6 (binary32), then for each eigenvector the codes of xi_it / s_i
    (binary32 quotient) with coordinate 2t in the low and 2t + 1 in the high nibble of byte t.
    Returns uint8 [B, Hkv, nb, fp4_block_bytes(d)]."""
    assert shape.dtype == "bf16"
    B, Hkv, nb, d, r = shape.batch, shape.n_kv_heads, shape.n_blocks, shape.head_dim, COBS_RANK
    C = np.asarray(Kcov, np.uint16).reshape(B, Hkv, nb, 1 + r, d)
    out = np.zeros((B, Hkv, nb, fp4_block_bytes(d)), np.uint8)
    out[..., :2 * d] = C[:, :, :, 0].copy().view(np.uint8).reshape(B, Hkv, nb, 2 * d)
    xi = widen("bf16", C[:, :, :, 1:]).astype(np.float32)  # exact
    for b in range(B):
        for j in range(Hkv):
            for blk in range(nb):
                for i in range(r):
                    x = xi[b, j, blk, i]
                    sc = np.float32(np.abs(x).max()) / np.float32(6.0)
                    out[b, j, blk, 2 * d + 4 * i:2 * d + 4 * i + 4] = np.frombuffer(np.float32(sc).tobytes(), np.uint8)
                    codes = [e2m1_code(np.float32(v) / sc) if sc > 0 else 0 for v in x]
                    base = 2 * d + 4 * r + i * d // 2
                    for t in range(d // 2):
                        out[b, j, blk, base + t] = codes[2 * t] | (codes[2 * t + 1] << 4)
    return out


def cov4_unpack(shape: Shape, packed):
    """Mean keys (fp64) [B, Hkv, nb, d] and decoded eigenvectors s_i x E2M1(code) (fp64)
    [B, Hkv, nb, r, d] of FP4 descriptors."""
    B, Hkv, nb, d, r = shape.batch, shape.n_kv_heads, shape.n_blocks, shape.head_dim, COBS_RANK
    P = np.asarray(packed, np.uint8).reshape(B, Hkv, nb, fp4_block_bytes(d))
    mean = widen("bf16", P[..., :2 * d].copy().view(np.uint16))
    scales = P[..., 2 * d:2 * d + 4 * r].copy().view(np.float32).astype(np.float64)  # [B, Hkv, nb, r]
    codes = P[..., 2 * d + 4 * r:].reshape(B, Hkv, nb, r, d // 2)
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(B, Hkv, nb, r, d)
    mag = np.asarray(E2M1)[nib & 7]
    val = np.where(nib & 8, -mag, mag)
    return mean, scales[..., None] * val


def cobs2_fp4_logits(shape: Shape, q, packed):
    """Second-order block logits [B, Hq, nb] from FP4 descriptors: the formula of
    cobs2_logits with the decoded eigenvectors."""
    B, Hq, Hkv, d, nb = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.n_blocks
    G = Hq // Hkv
    qf = widen(shape, _stored(shape, q, (B, Hq, d)))
    mean, xi = cov4_unpack(shape, packed)
    scale = shape.scale if shape.scale else 1.0 / math.sqrt(d)
    counts = np.array([min(shape.block_size, shape.n_tokens - i * shape.block_size) for i in range(nb)], np.float64)
    out = np.empty((B, Hq, nb), np.float64)
    for h in range(Hq):
        m1 = np.einsum("bd,bkd->bk", qf[:, h], mean[:, h // G])
        m2 = np.einsum("bd,bkrd->bkr", qf[:, h], xi[:, h // G])
        out[:, h] = scale * m1 + np.log(counts) + 0.5 * scale * scale * (m2 ** 2).sum(-1)
    return out


def sub_padded(s_dim: int) -> int:
    """Stored length of a query-subspace eigenvector: s rounded up to whole 16-byte chunks of
    bfloat16 (8 elements), the padding zero."""
    return -(-s_dim // 8) * 8


def cov_sub_factors(shape: Shape, K, U, rank: int = COBS_RANK):
    """Query-subspace covariance factors of "COBS: Cumulant Order Block Sparse Attention"
    (section on keeping the covariance only within the query subspace): U [Hkv, d, s] holds
    the top s eigenvectors of the queries' second moment for each KV head (the caller's
    basis); per block B_b = U^T Sigma_b U (s x s), Sigma_b the within-block key covariance
    (1/c) sum_i (k_i - kbar)(k_i - kbar)^T, and its top `rank` scaled eigenvectors
    xi_i = sqrt(mu_i) v_i, largest first, each signed so that its largest-magnitude
    coordinate is positive.  fp64, unrounded: [B, Hkv, nb, rank, s]."""
    B, Hkv, n, d, L, nb = shape.batch, shape.n_kv_heads, shape.n_tokens, shape.head_dim, shape.block_size, \
        shape.n_blocks
    Kf = widen(shape, _stored(shape, K, (B, Hkv, n, d)))
    U = np.asarray(U, np.float64)
    s_dim = U.shape[-1]
    assert U.shape == (Hkv, d, s_dim)
    xi = np.zeros((B, Hkv, nb, rank, s_dim), np.float64)
    for b in range(B):
        for j in range(Hkv):
            for blk in range(nb):
                X = Kf[b, j, blk * L:min(n, (blk + 1) * L)]
                Y = (X - X.mean(axis=0)) @ U[j]  # centred keys in the query subspace
                mu, V = np.linalg.eigh(Y.T @ Y / X.shape[0])  # ascending
                for i in range(min(rank, s_dim)):
                    v = V[:, s_dim - 1 - i]
                    v = v if v[np.argmax(np.abs(v))] > 0 else -v
                    xi[b, j, blk, i] = math.sqrt(max(mu[s_dim - 1 - i], 0.0)) * v
    return xi


def cov_sub_build(shape: Shape, K, U, Kbar=None, rank: int = COBS_RANK):
    """Stored query-subspace descriptor [B, Hkv, nb, d + rank * sub_padded(s)] in the storage
    dtype: the mean key (the bits of kv_summary_build), then the `rank` factors of
    cov_sub_factors, each rounded once and zero-padded to sub_padded(s) elements."""
    B, Hkv, nb, d = shape.batch, shape.n_kv_heads, shape.n_blocks, shape.head_dim
    if Kbar is None:
        Kbar, _ = kv_summary_build(shape, K, K)
    xi = cov_sub_factors(shape, K, U, rank)
    s_dim = xi.shape[-1]
    sp = sub_padded(s_dim)
    out = np.zeros((B, Hkv, nb, d + rank * sp), shape.np_dtype)
    out[..., :d] = np.asarray(Kbar).reshape(B, Hkv, nb, d)
    padded = np.zeros((B, Hkv, nb, rank, sp), np.float64)
    padded[..., :s_dim] = xi
    out[..., d:] = store_array(shape, padded).reshape(B, Hkv, nb, rank * sp)
    return out


def cov_sub_unpack(shape: Shape, Kcs, s_dim: int, rank: int = COBS_RANK):
    """Mean keys [B, Hkv, nb, d] and factors [B, Hkv, nb, rank, s] (fp64) of a stored
    query-subspace descriptor."""
    B, Hkv, nb, d = shape.batch, shape.n_kv_heads, shape.n_blocks, shape.head_dim
    sp = sub_padded(s_dim)
    C = widen(shape, np.asarray(Kcs).reshape(B, Hkv, nb, d + rank * sp))
    return C[..., :d], C[..., d:].reshape(B, Hkv, nb, rank, sp)[..., :s_dim]


def cobs2_sub_logits(shape: Shape, q, Kcs, U):
    """Second-order block logits [B, Hq, nb] from query-subspace descriptors: the cumulant
    estimate truncated at second order with the covariance kept in the subspace,
    scale q.kbar_b + ln c_b + (1/2) scale^2 sum_i (qt . xi_i)^2 with qt = U^T q the query's
    coordinates in the subspace of its KV head."""
    B, Hq, Hkv, d, nb = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.n_blocks
    G = Hq // Hkv
    U = np.asarray(U, np.float64)
    s_dim = U.shape[-1]
    qf = widen(shape, _stored(shape, q, (B, Hq, d)))
    mean, xi = cov_sub_unpack(shape, Kcs, s_dim)
    scale = shape.scale if shape.scale else 1.0 / math.sqrt(d)
    counts = np.array([min(shape.block_size, shape.n_tokens - i * shape.block_size) for i in range(nb)], np.float64)
    out = np.empty((B, Hq, nb), np.float64)
    for h in range(Hq):
        qt = qf[:, h] @ U[h // G]  # [B, s]
        m1 = np.einsum("bd,bkd->bk", qf[:, h], mean[:, h // G])
        m2 = np.einsum("bs,bkrs->bkr", qt, xi[:, h // G])
        out[:, h] = scale * m1 + np.log(counts) + 0.5 * scale * scale * (m2 ** 2).sum(-1)
    return out


def sub4_padded(s_dim: int) -> int:
    """Coordinates per FP4 query-subspace factor: s rounded up to 32 (16 bytes of codes)."""
    return -(-s_dim // 32) * 32


def sub4_block_bytes(d: int, s_dim: int, rank: int = COBS_RANK) -> int:
    """Bytes per block of the FP4 query-subspace descriptor: the bfloat16 mean key, one fp32
    scale per factor, then the factors' 4-bit codes (two per byte, zero codes past s)."""
    return 2 * d + 4 * rank + rank * sub4_padded(s_dim) // 2


def cov_sub4_pack(shape: Shape, Kcs, s_dim: int):
    """FP4 storage of query-subspace descriptors (the FP4 quantisation of the COBS page applied
    to the subspace factors), from the stored bfloat16 descriptors Kcs: per block the mean row
    (its bits), the scales s_i = max_t |xi_it| / 6 (binary32), then for each factor the codes
    of xi_it / s_i (binary32 quotient) for t < s and zero codes up to sub4_padded(s), coordinate
    2t in the low and 2t + 1 in the high nibble of byte t.  Returns uint8
    [B, Hkv, nb, sub4_block_bytes(d, s)]."""
    assert shape.dtype == "bf16"
    B, Hkv, nb, d, r = shape.batch, shape.n_kv_heads, shape.n_blocks, shape.head_dim, COBS_RANK
    sp, sf = sub_padded(s_dim), sub4_padded(s_dim)
    C = np.asarray(Kcs, np.uint16).reshape(B, Hkv, nb, d + r * sp)
    out = np.zeros((B, Hkv, nb, sub4_block_bytes(d, s_dim)), np.uint8)
    out[..., :2 * d] = C[..., :d].copy().view(np.uint8).reshape(B, Hkv, nb, 2 * d)
    xi = widen("bf16", C[..., d:].reshape(B, Hkv, nb, r, sp)[..., :s_dim]).astype(np.float32)  # exact
    for b in range(B):
        for j in range(Hkv):
            for blk in range(nb):
                for i in range(r):
                    x = xi[b, j, blk, i]
                    sc = np.float32(np.abs(x).max()) / np.float32(6.0)
                    out[b, j, blk, 2 * d + 4 * i:2 * d + 4 * i + 4] = np.frombuffer(np.float32(sc).tobytes(), np.uint8)
                    codes = [e2m1_code(np.float32(v) / sc) if sc > 0 else 0 for v in x] + [0] * (sf - s_dim)
                    base = 2 * d + 4 * r + i * sf // 2
                    for t in range(sf // 2):
                        out[b, j, blk, base + t] = codes[2 * t] | (codes[2 * t + 1] << 4)
    return out


def cov_sub4_unpack(shape: Shape, packed, s_dim: int):
    """Mean keys (fp64) [B, Hkv, nb, d] and decoded factors s_i x E2M1(code) (fp64)
    [B, Hkv, nb, r, s] of FP4 query-subspace descriptors."""
    B, Hkv, nb, d, r = shape.batch, shape.n_kv_heads, shape.n_blocks, shape.head_dim, COBS_RANK
    sf = sub4_padded(s_dim)
    P = np.asarray(packed, np.uint8).reshape(B, Hkv, nb, sub4_block_bytes(d, s_dim))
    mean = widen("bf16", P[..., :2 * d].copy().view(np.uint16))
    scales = P[..., 2 * d:2 * d + 4 * r].copy().view(np.float32).astype(np.float64)
    codes = P[..., 2 * d + 4 * r:].reshape(B, Hkv, nb, r, sf // 2)
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(B, Hkv, nb, r, sf)[..., :s_dim]
    mag = np.asarray(E2M1)[nib & 7]
    return mean, scales[..., None] * np.where(nib & 8, -mag, mag)


def cobs2_sub4_logits(shape: Shape, q, packed, U):
    """The logits of cobs2_sub_logits from FP4 query-subspace descriptors (decoded factors)."""
    B, Hq, Hkv, d, nb = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.n_blocks
    G = Hq // Hkv
    U = np.asarray(U, np.float64)
    qf = widen(shape, _stored(shape, q, (B, Hq, d)))
    mean, xi = cov_sub4_unpack(shape, packed, U.shape[-1])
    scale = shape.scale if shape.scale else 1.0 / math.sqrt(d)
    counts = np.array([min(shape.block_size, shape.n_tokens - i * shape.block_size) for i in range(nb)], np.float64)
    out = np.empty((B, Hq, nb), np.float64)
    for h in range(Hq):
        qt = qf[:, h] @ U[h // G]
        m1 = np.einsum("bd,bkd->bk", qf[:, h], mean[:, h // G])
        m2 = np.einsum("bs,bkrs->bkr", qt, xi[:, h // G])
        out[:, h] = scale * m1 + np.log(counts) + 0.5 * scale * scale * (m2 ** 2).sum(-1)
    return out


def block_logits(shape: Shape, mode: int, q, keys):
    """Per-query-head block logits [B, Hq, nb]: first-order summary score, exact ln m_b, or the
    largest logit over the block's key box."""
    if mode == COBS2:
        return cobs2_logits(shape, q, keys)
    if mode == COBS2_FP4:
        return cobs2_fp4_logits(shape, q, keys)
    rows = {SUMMARY: shape.n_blocks, EXACT_MASS: shape.n_tokens, BOX: 2 * shape.n_blocks}[mode]
    q = _stored(shape, q, (shape.batch, shape.n_q_heads, shape.head_dim))
    if mode == BOX:  # [B, Hkv, nb, 2, d] is [B, Hkv, 2 nb, d] in memory
        keys = np.asarray(keys)
        if keys.ndim == 5:
            keys = keys.reshape(shape.batch, shape.n_kv_heads, rows, shape.head_dim)
    keys = _stored(shape, keys, (shape.batch, shape.n_kv_heads, rows, shape.head_dim))
    out = np.empty((shape.batch, shape.n_q_heads, shape.n_blocks), np.float64)
    _check(_load().oracle_block_logits(ctypes.byref(shape.c()), mode, _ptr(q), _ptr(keys), _ptr(out)),
           "block_logits")
    return out


def group_score(shape: Shape, logits):
    """Group block score [B, Hkv, nb] (log of the sum of per-head normalised masses for G > 1)."""
    logits = np.ascontiguousarray(logits, np.float64)
    assert logits.shape == (shape.batch, shape.n_q_heads, shape.n_blocks)
    out = np.empty((shape.batch, shape.n_kv_heads, shape.n_blocks), np.float64)
    _check(_load().oracle_group_score(ctypes.byref(shape.c()), _ptr(logits), _ptr(out)), "group_score")
    return out


def block_score(shape: Shape, mode: int, q, keys):
    if mode == PROXY_ERROR:
        return proxy_error_score(shape, q, keys)
    return group_score(shape, block_logits(shape, mode, q, keys))


def topk_select(scores, k: int):
    """Top-k of each row of a 2-D (or [B, Hkv, nb]) score array.

    Returns (sel, margin): sel [..., min(k, nb)] int32 ascending, margin [...] fp64
    = score_(k) - score_(k+1) in (score desc, index asc) order (inf if all kept)."""
    scores = np.ascontiguousarray(scores, np.float64)
    lead, nb = scores.shape[:-1], scores.shape[-1]
    rows = int(np.prod(lead)) if lead else 1
    kk = min(k, nb)
    sel = np.empty(lead + (kk,), np.int32)
    margin = np.empty(lead, np.float64)
    _check(_load().oracle_topk(rows, nb, k, _ptr(scores), _ptr(sel), _ptr(margin)), "topk")
    return sel, margin


def sparse_decode_attn(shape: Shape, q, K, V, Kbar, Vbar, sel, proxies: bool,
                       tok_idx=None, tok_logw=None):
    """Attention over exact tokens of the kept blocks, weighted tokens and proxies."""
    kv = (shape.batch, shape.n_kv_heads, shape.n_tokens, shape.head_dim)
    q = _stored(shape, q, (shape.batch, shape.n_q_heads, shape.head_dim))
    K, V = _stored(shape, K, kv), _stored(shape, V, kv)
    if proxies:
        sm = (shape.batch, shape.n_kv_heads, shape.n_blocks, shape.head_dim)
        Kbar, Vbar = _stored(shape, Kbar, sm), _stored(shape, Vbar, sm)
    else:
        Kbar = Vbar = None
    sel = np.ascontiguousarray(sel, np.int32)
    k = sel.shape[-1]
    assert sel.shape == (shape.batch, shape.n_kv_heads, k)
    m = 0
    if tok_idx is not None:
        tok_idx = np.ascontiguousarray(tok_idx, np.int32)
        tok_logw = np.ascontiguousarray(tok_logw, np.float32)
        m = tok_idx.shape[-1]
        assert tok_idx.shape == tok_logw.shape == (shape.batch, shape.n_kv_heads, m)
    out = np.empty((shape.batch, shape.n_q_heads, shape.head_dim), np.float64)
    lse = np.empty((shape.batch, shape.n_q_heads), np.float64)
    _check(_load().oracle_attend(ctypes.byref(shape.c()), _ptr(q), _ptr(K), _ptr(V), _ptr(Kbar), _ptr(Vbar),
                                 _ptr(sel), k, _ptr(tok_idx), _ptr(tok_logw), m, 1 if proxies else 0,
                                 _ptr(out), _ptr(lse)), "attend")
    return out, lse


def dense_decode_attn(shape: Shape, q, K, V):
    kv = (shape.batch, shape.n_kv_heads, shape.n_tokens, shape.head_dim)
    q = _stored(shape, q, (shape.batch, shape.n_q_heads, shape.head_dim))
    K, V = _stored(shape, K, kv), _stored(shape, V, kv)
    out = np.empty((shape.batch, shape.n_q_heads, shape.head_dim), np.float64)
    lse = np.empty((shape.batch, shape.n_q_heads), np.float64)
    _check(_load().oracle_dense(ctypes.byref(shape.c()), _ptr(q), _ptr(K), _ptr(V), _ptr(out), _ptr(lse)),
           "dense")
    return out, lse


def block_mass(shape: Shape, q, K, V, centroids: bool = False):
    """Exact ln m_b per query head [B, Hq, nb] and optionally the attention-weighted
    block centroids [B, Hq, nb, d]."""
    kv = (shape.batch, shape.n_kv_heads, shape.n_tokens, shape.head_dim)
    q = _stored(shape, q, (shape.batch, shape.n_q_heads, shape.head_dim))
    K, V = _stored(shape, K, kv), _stored(shape, V, kv)
    ln_m = np.empty((shape.batch, shape.n_q_heads, shape.n_blocks), np.float64)
    cen = np.empty((shape.batch, shape.n_q_heads, shape.n_blocks, shape.head_dim), np.float64) if centroids else None
    _check(_load().oracle_block_mass(ctypes.byref(shape.c()), _ptr(q), _ptr(K), _ptr(V), _ptr(ln_m), _ptr(cen)),
           "block_mass")
    return (ln_m, cen) if centroids else ln_m


def round_bf16(x: float) -> int:
    """The oracle's fp64 -> bfloat16 rounding (bit pattern)."""
    return int(_load().oracle_round_bf16(float(x)))


def widen(shape_or_dtype, a):
    """Stored array -> fp64 (exact)."""
    dt = shape_or_dtype.dtype if isinstance(shape_or_dtype, Shape) else shape_or_dtype
    if dt == "f32":
        return np.asarray(a, np.float32).astype(np.float64)
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Query-guided clusters ("OpenAttention reads 1% of the KV cache -- Count-aware
# tail proxy", section "Three helpers that make the proxy accurate")
# ---------------------------------------------------------------------------

def cluster_build(shape: Shape, K, V, U, init_idx, iters: int):
    """k-means of the keys projected on U [B, Hkv, d, r] (fp32), seeded at the tokens init_idx
    [B, Hkv, C], `iters` Lloyd rounds then a final assignment.  Returns a dict: assign [B, Hkv, n],
    order [B, Hkv, n], offsets [B, Hkv, C + 1], Kc, Vc [B, Hkv, C, d] (storage dtype), cent
    [B, Hkv, C, r] (fp64 final centroids)."""
    B, Hkv, n, d = shape.batch, shape.n_kv_heads, shape.n_tokens, shape.head_dim
    K, V = _stored(shape, K, (B, Hkv, n, d)), _stored(shape, V, (B, Hkv, n, d))
    U = np.ascontiguousarray(U, np.float32)
    init_idx = np.ascontiguousarray(init_idx, np.int32)
    r, C = U.shape[-1], init_idx.shape[-1]
    assert U.shape == (B, Hkv, d, r) and init_idx.shape == (B, Hkv, C)
    out = {"assign": np.empty((B, Hkv, n), np.int32), "order": np.empty((B, Hkv, n), np.int32),
           "offsets": np.empty((B, Hkv, C + 1), np.int32), "Kc": np.empty((B, Hkv, C, d), shape.np_dtype),
           "Vc": np.empty((B, Hkv, C, d), shape.np_dtype), "cent": np.empty((B, Hkv, C, r), np.float64)}
    _check(_load().oracle_cluster_build(ctypes.byref(shape.c()), C, r, iters, _ptr(K), _ptr(V), _ptr(U),
                                        _ptr(init_idx), _ptr(out["assign"]), _ptr(out["order"]),
                                        _ptr(out["offsets"]), _ptr(out["Kc"]), _ptr(out["Vc"]), _ptr(out["cent"])),
           "cluster_build")
    return out


def cluster_logits(shape: Shape, q, Kc, offsets):
    """[B, Hq, C]: scale q.Kc + ln count per cluster (-inf when empty)."""
    B, Hkv, d = shape.batch, shape.n_kv_heads, shape.head_dim
    offsets = np.ascontiguousarray(offsets, np.int32)
    C = offsets.shape[-1] - 1
    q = _stored(shape, q, (B, shape.n_q_heads, d))
    Kc = _stored(shape, Kc, (B, Hkv, C, d))
    out = np.empty((B, shape.n_q_heads, C), np.float64)
    _check(_load().oracle_cluster_logits(ctypes.byref(shape.c()), C, _ptr(q), _ptr(Kc), _ptr(offsets), _ptr(out)),
           "cluster_logits")
    return out


def cluster_score(shape: Shape, q, Kc, offsets):
    """Cluster scores [B, Hkv, C]: the group rule of block_score over the cluster logits."""
    lg = cluster_logits(shape, q, Kc, offsets)
    C = lg.shape[-1]
    gs = Shape(shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, C, 1, shape.dtype, shape.scale)
    return group_score(gs, lg)


def cluster_attend(shape: Shape, q, K, V, Kc, Vc, order, offsets, sel, proxies: bool):
    """Attention over every token of the selected clusters and a proxy per other cluster."""
    B, Hkv, n, d = shape.batch, shape.n_kv_heads, shape.n_tokens, shape.head_dim
    offsets = np.ascontiguousarray(offsets, np.int32)
    C = offsets.shape[-1] - 1
    q = _stored(shape, q, (B, shape.n_q_heads, d))
    K, V = _stored(shape, K, (B, Hkv, n, d)), _stored(shape, V, (B, Hkv, n, d))
    Kc, Vc = _stored(shape, Kc, (B, Hkv, C, d)), _stored(shape, Vc, (B, Hkv, C, d))
    order = np.ascontiguousarray(order, np.int32)
    sel = np.ascontiguousarray(sel, np.int32)
    k = sel.shape[-1]
    out = np.empty((B, shape.n_q_heads, d), np.float64)
    lse = np.empty((B, shape.n_q_heads), np.float64)
    _check(_load().oracle_cluster_attend(ctypes.byref(shape.c()), C, _ptr(q), _ptr(K), _ptr(V), _ptr(Kc), _ptr(Vc),
                                         _ptr(order), _ptr(offsets), _ptr(sel), k, 1 if proxies else 0, _ptr(out),
                                         _ptr(lse)), "cluster_attend")
    return out, lse
