"""Block-sparse attention as its plain definition (float64).

BSA-DiT §4.1: for every query block only the KV blocks listed for it are
visited; BSA-DiT §4.3: a skipped block behaves as if its scores were -inf, so
the softmax normaliser runs over the active keys only.  The result of a
block-sparse FlashAttention is therefore exactly (up to rounding)

    O = softmax(scale * Q K^T + M) V,   LSE = log sum_c exp(scale * q.k_c + M_c)

with M = 0 on keys whose block is listed for the query's block (and whose
index is < N) and M = -inf elsewhere.  That definition is what this module
computes, one query block at a time, over all N keys.

Readings where the pages are silent:
* a row with no active key (possible only for an empty CSR row) has O = 0 and
  LSE = -inf;
* LSE is the natural log and includes `scale`;
* query rows >= N do not exist (the last block may be partial).
"""
from __future__ import annotations

import numpy as np

__all__ = ["scores", "apply_mask", "softmax_stats", "masked_attention",
           "active_blocks", "block_sparse_attention", "dense_attention"]


def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """scale * q k^T for q [Nq, D], k [Nk, D]."""
    return scale * (q @ k.T)


def apply_mask(s: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Scores of keys that are not allowed become -inf (BSA-DiT §4.3)."""
    return np.where(allowed, s, -np.inf)


def softmax_stats(s: np.ndarray):
    """Row-wise softmax probabilities and natural-log LSE of masked scores.

    Uses the usual max shift (exact in real arithmetic).  Rows that are -inf
    everywhere give p = 0 and LSE = -inf.
    """
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    p = e / l_safe[:, None]
    lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return p, lse


def masked_attention(q, k, v, allowed, scale):
    """O, LSE of softmax(scale q k^T with -inf where not allowed) v."""
    s = apply_mask(scores(q, k, scale), allowed)
    p, lse = softmax_stats(s)
    return p @ v, lse


def active_blocks(row_ptr, col_idx, r):
    """Set of KV blocks listed for CSR row r (order and duplicates irrelevant)."""
    return np.unique(np.asarray(col_idx[row_ptr[r]:row_ptr[r + 1]], dtype=np.int64))


def _as64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def block_sparse_attention(q, k, v, row_ptr, col_idx, block, scale, rows=None):
    """Oracle O [B,H,N,D] and LSE [B,H,N] for a per-query-block CSR index.

    q, k, v: [B,H,N,D] (torch bf16 or numpy); row_ptr [B*H*nb+1], col_idx [nnz]
    with CSR row r = (b*H + h)*nb + i.  If `rows` is given, only those CSR rows
    are evaluated; the other outputs are NaN.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, D = q.shape
    nb = (N + block - 1) // block
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col_idx = np.asarray(col_idx, dtype=np.int64)
    assert row_ptr.shape[0] == B * H * nb + 1
    O = np.full((B, H, N, D), np.nan)
    L = np.full((B, H, N), np.nan)
    key_block = np.arange(N) // block
    todo = range(B * H * nb) if rows is None else rows
    for r in todo:
        bh, i = divmod(int(r), nb)
        b, h = divmod(bh, H)
        a0, a1 = i * block, min(N, (i + 1) * block)
        allowed_keys = np.isin(key_block, active_blocks(row_ptr, col_idx, r))
        allowed = np.broadcast_to(allowed_keys, (a1 - a0, N))
        o, lse = masked_attention(q[b, h, a0:a1], k[b, h], v[b, h], allowed, scale)
        O[b, h, a0:a1] = o
        L[b, h, a0:a1] = lse
    return O, L


def dense_attention(q, k, v, scale):
    """Unmasked softmax(scale q k^T) v and LSE per (b, h)."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, D = q.shape
    O = np.empty((B, H, N, D))
    L = np.empty((B, H, N))
    allowed = np.ones((N, N), dtype=bool)
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = masked_attention(q[b, h], k[b, h], v[b, h], allowed, scale)
    return O, L
