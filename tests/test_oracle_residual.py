"""Pins of the residual-compensation oracle (CPU): the anchor identity, zero drift,
the all-ones CSR and the gain under slow drift (oracle/residual.py, from the page on
the quality gap of sparse attention in diffusion transformers, sections on reusing
exact selection and on residual compensation)."""
import numpy as np

import workloads as W
from oracle import attention as A
from oracle import residual as R


def _csr(nb, rows, keep, seed):
    rng = np.random.default_rng(seed)
    cols = []
    for r in range(rows):
        i = r % nb
        c = set(rng.choice(nb, keep, replace=False).tolist()) | {i}
        cols.append(sorted(c))
    rp = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    return rp, np.concatenate(cols).astype(np.int32)


def _setup(eps, steps=3, N=96, block=32, D=16):
    qkv = W.drifting_qkv(4, steps, eps, 1, 2, N, D, block)
    nb = N // block
    rp, ci = _csr(nb, 2 * nb, 1, 9)
    return R.anchor_and_reuse(qkv, rp, ci, block, 0.25), rp, ci, qkv


def test_anchor_step_is_exact():
    out, _, _, _ = _setup(0.05)
    od, os_, oc = out[0]
    np.testing.assert_allclose(oc, od, rtol=0, atol=1e-12)
    assert np.abs(os_ - od).max() > 1e-3      # the sparse output alone is not dense


def test_zero_drift_reuses_exactly():
    out, _, _, _ = _setup(0.0)
    for od, _, oc in out:
        np.testing.assert_allclose(oc, od, rtol=0, atol=1e-12)


def test_all_ones_csr_has_zero_residual():
    qkv = W.drifting_qkv(1, 1, 0.0, 1, 1, 64, 8, 32)
    q, k, v = qkv[0]
    rp = np.array([0, 2, 4], np.int32)
    ci = np.array([0, 1, 0, 1], np.int32)
    od, _ = A.dense_attention(q, k, v, 0.3)
    os_, _ = A.block_sparse_attention(q, k, v, rp, ci, 32, 0.3)
    assert np.abs(R.residual(od, os_)).max() < 1e-12


def test_small_drift_compensation_beats_sparse():
    """Under slow drift the cached residual brings the output closer to dense attention
    than the sparse output alone."""
    out, _, _, _ = _setup(0.02, steps=4)
    for od, os_, oc in out[1:]:
        assert np.linalg.norm(oc - od) < 0.5 * np.linalg.norm(os_ - od)


def test_residual_sign():
    a = np.array([1.0, 2.0, -3.0])
    b = np.array([0.5, 2.5, -1.0])
    assert R.residual(a, b).tolist() == [0.5, -0.5, -2.0]
    assert R.compensate(b, R.residual(a, b)).tolist() == a.tolist()
