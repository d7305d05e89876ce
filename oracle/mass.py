"""Exact attention mass per block pair and the block oracle (float64).

Test infrastructure: only the tests, the smoke entry point and the benchmark's
CPU baseline use this module; the library never does.

Page "Can sparse attention close the quality gap in diffusion transformers"
(wispaper.ai summary of MC-Sparse):
* section "the quality gap has three separable sources" and section "the oracle
  analysis bounds what sparsity can recover": sparse attention is compared, at
  the same attention density, with oracles that use the exact dense attention
  probabilities to keep as much attention mass as possible; the block oracle
  chooses KV blocks for every query block;
* section "token-level selection needs tile-aligned query groups": exact
  selection needs the attention scores, which a FlashAttention pass does not
  expose, hence two passes (first the dense softmax normaliser, then the
  probabilities themselves).

Definitions written out here (the plain reading of those sections):
* P = softmax(scale q k^T) over all N keys, per (batch, head): the dense
  attention probabilities;
* mass[b,h,i,j] = sum over queries t of block i and keys c of block j (t, c < N)
  of P[t, c].  Every query's probabilities sum to one, so a row of the mass
  matrix sums to the number of queries in block i;
* the block oracle at equal density keeps, for every row (b, h, i), as many KV
  blocks as a given CSR row, the ones of largest mass (ties to the lower block
  index), listed ascending;
* the retained mass of a CSR row is the sum of mass over its blocks; divided by
  the row's query count it is the mean attention probability its queries keep.
"""
from __future__ import annotations

import numpy as np

__all__ = ["dense_probabilities", "block_mass", "oracle_csr", "retained_mass"]


def _as64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def dense_probabilities(q, k, scale: float) -> np.ndarray:
    """P = softmax(scale q k^T) for q [Nq, D], k [Nk, D] (max-shifted, exact in reals)."""
    s = scale * (_as64(q) @ _as64(k).T)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def block_mass(q, k, block: int, scale: float) -> np.ndarray:
    """mass [B, H, nb, nb]: block sums of the dense probabilities of every head."""
    q, k = _as64(q), _as64(k)
    B, H, N, _ = q.shape
    nb = -(-N // block)
    pad = nb * block - N
    out = np.empty((B, H, nb, nb))
    for b in range(B):
        for h in range(H):
            p = dense_probabilities(q[b, h], k[b, h], scale)
            p = np.pad(p, ((0, pad), (0, pad)))
            out[b, h] = p.reshape(nb, block, nb, block).sum(axis=(1, 3))
    return out


def oracle_csr(mass: np.ndarray, row_ptr) -> np.ndarray:
    """col_idx of the block oracle: for row r, the row_ptr[r+1]-row_ptr[r] blocks of
    largest mass[r] (ties to the lower block), ascending."""
    m = np.asarray(mass, dtype=np.float64).reshape(-1, mass.shape[-1])
    rp = np.asarray(row_ptr, dtype=np.int64)
    nb = m.shape[1]
    cols = []
    for r in range(m.shape[0]):
        n = int(rp[r + 1] - rp[r])
        assert 0 <= n <= nb, "a CSR row longer than the block count"
        order = np.lexsort((np.arange(nb), -m[r]))  # mass descending, then index ascending
        cols.append(np.sort(order[:n]))
    return np.concatenate(cols).astype(np.int32) if cols else np.zeros(0, np.int32)


def retained_mass(mass: np.ndarray, row_ptr, col_idx) -> np.ndarray:
    """Per CSR row: the mass of its listed blocks (a block listed twice counts once)."""
    m = np.asarray(mass, dtype=np.float64).reshape(-1, mass.shape[-1])
    rp = np.asarray(row_ptr, dtype=np.int64)
    ci = np.asarray(col_idx, dtype=np.int64)
    out = np.zeros(m.shape[0])
    for r in range(m.shape[0]):
        cols = np.unique(ci[rp[r]:rp[r + 1]])
        out[r] = m[r, cols].sum()
    return out
