"""Caller-side query statistics: the basis of the query-guided cluster build ("OpenAttention
reads 1% of the KV cache -- Count-aware tail proxy", section "Three helpers that make the proxy
accurate": keys are projected onto the top eigenvectors of the queries) and of the
query-subspace descriptors ("COBS: Cumulant Order Block Sparse Attention", section on keeping
the covariance within the query subspace), and the cluster seeds.  The library takes them as
inputs; the tests and the benchmark make them here, from the seeded prefill queries of the
workload generator."""
import numpy as np


def query_basis(queries: np.ndarray, r: int) -> np.ndarray:
    """[..., N, d] prefill queries -> [..., d, r] float32: the r eigenvectors of the queries'
    second moment (1/N) sum q q^T with the largest eigenvalues, largest first, each signed so
    that its largest-magnitude coordinate is positive."""
    lead, (N, d) = queries.shape[:-2], queries.shape[-2:]
    Qf = queries.reshape(-1, N, d)
    out = np.empty((Qf.shape[0], d, r), np.float32)
    for i, Q in enumerate(Qf):
        M = Q.T @ Q / N
        lam, U = np.linalg.eigh(M)  # ascending
        top = U[:, ::-1][:, :r].copy()
        for c in range(r):
            if top[np.argmax(np.abs(top[:, c])), c] < 0:
                top[:, c] = -top[:, c]
        out[i] = top.astype(np.float32)
    return out.reshape(*lead, d, r)


def seed_tokens(B: int, Hkv: int, n: int, C: int) -> np.ndarray:
    """The tokens whose projections start the C centroids: evenly spaced, c n / C."""
    return np.broadcast_to((np.arange(C, dtype=np.int64) * n // C).astype(np.int32), (B, Hkv, C)).copy()


def pooled_query_basis(queries: np.ndarray, s_dim: int) -> np.ndarray:
    """[B, Hkv, N, d] prefill queries -> [Hkv, d, s] float32: per KV head the query basis of
    its queries pooled over the batch (the query statistics of a layer's KV head, shared by
    every sequence)."""
    B, Hkv, N, d = queries.shape
    pooled = np.ascontiguousarray(np.transpose(queries, (1, 0, 2, 3)).reshape(Hkv, B * N, d))
    return query_basis(pooled, s_dim)
