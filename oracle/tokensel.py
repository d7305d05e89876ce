"""Token-level KV selection with tile-aligned query groups (float64).

Test infrastructure: only the tests, the smoke entry point and the benchmark's
CPU baseline use this module; the library never does.

Page "Can sparse attention close the quality gap in diffusion transformers"
(wispaper.ai summary of MC-Sparse), section "token-level selection needs
tile-aligned query groups":
* KV tokens are selected one by one for each query group, across block
  boundaries, and gathered by index (not repacked into blocks);
* because every head has its own keys and values, an efficient tile batches the
  queries of one head: C similar queries form a group;
* groups of equal size come from the median-split version of principal-direction
  divisive partitioning: each group is projected on its principal direction and
  cut at the median, recursively;
* exact token selection needs the attention scores (a two-pass kernel).

Readings (the page leaves the steps open; these are the plainest ones):
* the principal direction is taken by POWER_ITERS steps of power iteration on
  the group's centred queries, from the start vector u[d] = 1 + d / D
  (normalised) — an iteration, so this module takes those exact steps;
* a group of g*C queries (g > 1) is cut into floor(g/2)*C and the rest: the
  queries of smallest projection (ties to the lower token index) go first —
  the median when g is even, the nearest cut that keeps tile-sized groups when it
  is odd; groups are numbered depth first, first part first;
* a group's selected tokens are the k of largest mass, the mass of token c being
  the sum over the group's queries t of the dense probability P[t, c] (ties to
  the lower token index), listed ascending;
* gathered attention: each query attends to exactly its group's tokens.
"""
from __future__ import annotations

import numpy as np

from . import attention as A
from . import mass as M

__all__ = ["POWER_ITERS", "start_vector", "principal_direction", "median_split_groups", "token_mass",
           "select_tokens", "gathered_attention"]

POWER_ITERS = 8


def _as64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def start_vector(D: int) -> np.ndarray:
    """The power iteration's start vector u[d] = 1 + d / D (not normalised)."""
    return 1.0 + np.arange(D) / D


def principal_direction(x: np.ndarray, iters: int | None = None) -> np.ndarray:
    """Unit vector after `iters` (default POWER_ITERS) power-iteration steps
    v <- X^T (X v) / |.| on the centred rows X of x, from start_vector(D)."""
    iters = POWER_ITERS if iters is None else iters
    xc = x - x.mean(axis=0)
    D = x.shape[1]
    v = start_vector(D)
    v = v / np.linalg.norm(v)
    for _ in range(iters):
        w = xc.T @ (xc @ v)
        n = np.linalg.norm(w)
        if n == 0.0:
            break
        v = w / n
    return v


def median_split_groups(x, C: int, iters: int | None = None) -> np.ndarray:
    """Groups [N / C, C] of token indices (each row ascending) for queries x [N, D];
    N must be a multiple of C."""
    x = _as64(x)
    N = x.shape[0]
    assert N % C == 0, "query count must be a multiple of the group size"
    out = []

    def split(idx):
        g = idx.size // C
        if g == 1:
            out.append(np.sort(idx))
            return
        sub = x[idx]
        p = (sub - sub.mean(axis=0)) @ principal_direction(sub, iters)
        order = idx[np.lexsort((idx, p))]  # projection ascending, then token index
        cut = (g // 2) * C
        split(order[:cut])
        split(order[cut:])

    split(np.arange(N))
    return np.stack(out)


def token_mass(q, k, groups: np.ndarray, scale: float) -> np.ndarray:
    """[G, N]: for every group, the dense attention probability summed over its queries."""
    P = M.dense_probabilities(q, k, scale)
    return np.stack([P[g].sum(axis=0) for g in np.asarray(groups)])


def select_tokens(mass_g: np.ndarray, k: int) -> np.ndarray:
    """[G, k]: per group the k tokens of largest mass (ties to the lower index), ascending."""
    m = np.asarray(mass_g, dtype=np.float64)
    N = m.shape[1]
    return np.stack([np.sort(np.lexsort((np.arange(N), -row))[:k]) for row in m])


def gathered_attention(q, k, v, groups: np.ndarray, tokens: np.ndarray, scale: float):
    """O [N, D], LSE [N] when the queries of group g attend to exactly tokens[g]."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    N = q.shape[0]
    O = np.zeros_like(q)
    L = np.full(N, -np.inf)
    for g, toks in zip(np.asarray(groups), np.asarray(tokens)):
        allowed = np.zeros((len(g), k.shape[0]), dtype=bool)
        allowed[:, toks] = True
        O[g], L[g] = A.masked_attention(q[g], k, v, allowed, scale)
    return O, L
