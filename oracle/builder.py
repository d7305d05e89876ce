"""Mean-pool top-k block-mask builder, step by step (float64).

MC-Sparse summary, section "均值池化块打分漏掉高权重 token" (mean-pooled block
scoring misses high-weight tokens): the naive block-sparse selector represents
every query block and every KV block by the mean of its queries / keys, scores
each (query block, KV block) pair by the dot product of those means, and keeps
the highest-scoring KV blocks at a given attention density.  BSA-DiT §2.3
combines such a dynamic choice with a static structural prior, and BSA-DiT §5.3
lets every query block carry its own target count.

Steps, in that order:
 1. Pq, Pk = means over the valid tokens of each block (a partial last block
    averages only the tokens < N).
 2. Sblk = Pq Pk^T (unscaled dot products).
 3. K_i  = per-row budget: budgets[i] if given, else K(density) (see `budget`).
 4. sel_i = prior row i (per head or shared), plus block i if force_diag.
 5. fill  = max(0, K_i - |sel_i|) further columns, taken from the columns not
    in sel_i by descending score, ties to the lower column index.
 6. the row is sel_i plus the fill, listed in ascending column order.

Readings where the pages are silent or garbled (all listed in the design notes):
* K(density) = 0 for density <= 0, else clamp(floor(density*nb + 0.5), 1, nb);
* the diagonal and prior count toward K_i; a row keeps its whole prior even
  when the prior alone exceeds K_i ("fill to budget");
* gap_i = (lowest filled score) - (highest score left out), +inf when nothing
  was filled or nothing is left out: selections are only unique where the gap
  is positive, and the GPU is compared bit for bit where gap > 1e-4.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["mean_pool", "block_scores", "budget", "row_budgets", "prior_row",
           "select_row", "plan_counts", "build_mask"]


def _as64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def mean_pool(x, block: int) -> np.ndarray:
    """[B,H,N,D] -> [B,H,nb,D]: mean over the valid tokens of every block."""
    x = _as64(x)
    B, H, N, D = x.shape
    nb = (N + block - 1) // block
    out = np.empty((B, H, nb, D))
    for i in range(nb):
        a0, a1 = i * block, min(N, (i + 1) * block)
        out[:, :, i, :] = x[:, :, a0:a1, :].sum(axis=2) / (a1 - a0)
    return out


def block_scores(pq: np.ndarray, pk: np.ndarray) -> np.ndarray:
    """Sblk[b,h,i,j] = Pq[b,h,i,:] . Pk[b,h,j,:] (no scale)."""
    return pq @ np.swapaxes(pk, -1, -2)


def budget(nb: int, density: float) -> int:
    """Blocks per row for a target density: round half up, at least one if density > 0."""
    if density <= 0.0:
        return 0
    return int(min(nb, max(1, math.floor(density * nb + 0.5))))


def row_budgets(nb: int, density: float, budgets=None) -> np.ndarray:
    """Per-query-block target counts K_i (explicit budgets win over density)."""
    if budgets is not None:
        return np.clip(np.asarray(budgets, dtype=np.int64), 0, nb)
    return np.full(nb, budget(nb, density), dtype=np.int64)


def prior_row(prior, b: int, h: int, i: int, nb: int, force_diag: bool) -> np.ndarray:
    """Boolean [nb]: the static prior of row i (per head if 4-D), plus i if forced."""
    sel = np.zeros(nb, dtype=bool)
    if prior is not None:
        p = np.asarray(prior)
        sel |= (p[b, h, i] if p.ndim == 4 else p[i]).astype(bool)
    if force_diag:
        sel[i] = True
    return sel


def select_row(score_row: np.ndarray, sel: np.ndarray, k_i: int):
    """Columns of one row (ascending) and its gap, per steps 4-6."""
    nb = score_row.shape[0]
    fill = max(0, int(k_i) - int(sel.sum()))
    cand = np.flatnonzero(~sel)
    order = cand[np.lexsort((cand, -score_row[cand]))]  # score desc, then index asc
    chosen = order[:fill]
    left = order[fill:]
    if fill == 0 or left.size == 0:
        gap = math.inf
    else:
        gap = float(score_row[chosen[-1]] - score_row[left[0]])
    cols = np.sort(np.concatenate([np.flatnonzero(sel), chosen]))
    assert cols.size == np.unique(cols).size and cols.size <= nb
    return cols, gap


def plan_counts(B: int, H: int, nb: int, density: float, prior=None, budgets=None,
                force_diag: bool = True) -> np.ndarray:
    """Row counts max(|sel_i|, K_i) for every CSR row r = (b*H+h)*nb + i."""
    kk = row_budgets(nb, density, budgets)
    counts = np.empty(B * H * nb, dtype=np.int64)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                s = int(prior_row(prior, b, h, i, nb, force_diag).sum())
                counts[(b * H + h) * nb + i] = max(s, int(kk[i]))
    return counts


def build_mask(q, k, block: int, density: float, prior=None, budgets=None,
               force_diag: bool = True):
    """CSR (row_ptr int64 [B*H*nb+1], col_idx int64 [nnz]) and per-row gaps.

    Pooling and scores are only evaluated when some row needs a fill.
    """
    q = _as64(q) if not isinstance(q, np.ndarray) else q
    B, H, N, D = q.shape
    nb = (N + block - 1) // block
    kk = row_budgets(nb, density, budgets)
    need_scores = False
    sels = {}
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                sel = prior_row(prior, b, h, i, nb, force_diag)
                sels[(b, h, i)] = sel
                if kk[i] > sel.sum():
                    need_scores = True
    S = None
    if need_scores:
        S = block_scores(mean_pool(q, block), mean_pool(k, block))
    row_ptr = np.zeros(B * H * nb + 1, dtype=np.int64)
    cols_all, gaps = [], np.full(B * H * nb, math.inf)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                r = (b * H + h) * nb + i
                sel = sels[(b, h, i)]
                if S is None:
                    cols, gap = np.flatnonzero(sel), math.inf
                else:
                    cols, gap = select_row(S[b, h, i], sel, kk[i])
                cols_all.append(cols)
                gaps[r] = gap
                row_ptr[r + 1] = row_ptr[r] + cols.size
    col_idx = np.concatenate(cols_all).astype(np.int64) if cols_all else np.zeros(0, np.int64)
    return row_ptr, col_idx, gaps
