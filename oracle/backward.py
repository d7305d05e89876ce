"""Gradients of block-sparse attention (float64).

Test infrastructure: only the tests, the smoke entry point and the benchmark's
CPU baseline use this module; the library never does.

BSA-DiT §2.3 and §5.2 use block-sparse attention while training (static masks
fixed before training, routed masks learnt in it, and the train/inference
alignment of both), so gradients through the same CSR are needed; the pages
describe the forward only (§4.1, §4.3: listed blocks visited, skipped blocks as
-inf scores).

Reading: the backward is the exact gradient of the forward's plain definition

    O = softmax(scale * Q K^T + M) V      (M = 0 on listed keys < N, -inf elsewhere)

with respect to Q, K and V, for an incoming gradient dO of O (the LSE output
receives none).  By the chain rule, for a query row t and its active keys c:

    P[t, c]  = exp(scale * q_t . k_c - LSE_t)          (0 on inactive keys)
    dV       = P^T dO
    dP       = dO V^T
    delta_t  = sum_d dO[t, d] O[t, d]                  (= sum_c P[t, c] dP[t, c])
    dS       = P * (dP - delta)
    dQ       = scale * dS K,     dK = scale * dS^T Q

Rows with no active key have P = 0 and contribute nothing (their dQ is 0).  This
module takes exactly these steps, one query block at a time over all N keys.
"""
from __future__ import annotations

import numpy as np

from . import attention as A

__all__ = ["probabilities", "delta", "score_gradient", "block_sparse_backward"]


def _as64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def probabilities(q, k, allowed, scale):
    """P [Nq, Nk] and O-independent LSE [Nq] of the masked softmax (0 / -inf on empty rows)."""
    return A.softmax_stats(A.apply_mask(A.scores(q, k, scale), allowed))


def delta(do, o):
    """Row-wise sum_d dO[t, d] O[t, d]."""
    return (do * o).sum(axis=1)


def score_gradient(p, dp, dl):
    """dS = P * (dP - delta): the softmax's Jacobian applied to dP, row by row."""
    return p * (dp - dl[:, None])


def block_sparse_backward(q, k, v, row_ptr, col_idx, block, scale, do):
    """dQ, dK, dV [B,H,N,D] (float64) for the CSR forward of oracle.attention.

    q, k, v, do: [B,H,N,D] (torch bf16 or numpy); row_ptr [B*H*nb+1], col_idx [nnz],
    CSR row r = (b*H + h)*nb + i.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, H, N, D = q.shape
    nb = (N + block - 1) // block
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col_idx = np.asarray(col_idx, dtype=np.int64)
    assert row_ptr.shape[0] == B * H * nb + 1
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    key_block = np.arange(N) // block
    for r in range(B * H * nb):
        bh, i = divmod(r, nb)
        b, h = divmod(bh, H)
        a0, a1 = i * block, min(N, (i + 1) * block)
        allowed_keys = np.isin(key_block, A.active_blocks(row_ptr, col_idx, r))
        allowed = np.broadcast_to(allowed_keys, (a1 - a0, N))
        p, _ = probabilities(q[b, h, a0:a1], k[b, h], allowed, scale)
        o = p @ v[b, h]
        g = do[b, h, a0:a1]
        dv[b, h] += p.T @ g
        dp = g @ v[b, h].T
        ds = score_gradient(p, dp, delta(g, o))
        dq[b, h, a0:a1] = scale * (ds @ k[b, h])
        dk[b, h] += scale * (ds.T @ q[b, h, a0:a1])
    return dq, dk, dv
