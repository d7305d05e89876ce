"""Dense-sparse residual compensation across reuse steps (float64).

Test infrastructure: only the tests, the smoke entry point and the benchmark's
CPU baseline use this module; the library never does.

Page "Can sparse attention close the quality gap in diffusion transformers"
(wispaper.ai summary of MC-Sparse):
* section "reusing exact selection beats recomputing mean pooling": the exact
  selection is made only at anchor steps and reused at the following steps,
  because the attention pattern is stable between nearby denoising steps;
* section "residual compensation recovers the dropped tail": at an anchor step
  the residual between the dense and the sparse attention outputs is recorded,
  and at a reuse step the cached residual is added to the sparse output.

Written out (the plain reading): with O_dense(x) and O_sparse(x; C) the dense and
the block-sparse attention outputs for inputs x and CSR C,
    anchor step a:  C_a chosen (any selector), R = O_dense(x_a) - O_sparse(x_a; C_a);
    reuse step t:   O_t = O_sparse(x_t; C_a) + R.
At the anchor step itself O_a = O_dense(x_a) exactly.
"""
from __future__ import annotations

import numpy as np

from . import attention as A

__all__ = ["residual", "compensate", "anchor_and_reuse"]


def residual(o_dense, o_sparse) -> np.ndarray:
    """R = O_dense - O_sparse, element by element."""
    return np.asarray(o_dense, dtype=np.float64) - np.asarray(o_sparse, dtype=np.float64)


def compensate(o_sparse, r) -> np.ndarray:
    """O = O_sparse + R, element by element."""
    return np.asarray(o_sparse, dtype=np.float64) + np.asarray(r, dtype=np.float64)


def anchor_and_reuse(steps_qkv, row_ptr, col_idx, block: int, scale: float):
    """For inputs of several steps (step 0 the anchor): per step the dense output, the
    sparse output with the anchor's CSR, and the compensated output."""
    out = []
    r = None
    for t, (q, k, v) in enumerate(steps_qkv):
        od, _ = A.dense_attention(q, k, v, scale)
        os_, _ = A.block_sparse_attention(q, k, v, row_ptr, col_idx, block, scale)
        if t == 0:
            r = residual(od, os_)
        out.append((od, os_, compensate(os_, r)))
    return out
