"""Pins of the block-mass oracle (CPU): closed forms, brute force and optimality.

The oracle is `oracle/mass.py` (exact dense attention mass per block pair and
the block oracle at equal density, from the page on the quality gap of sparse
attention in diffusion transformers, sections on the three sources of the gap
and on what the oracle analysis bounds).
"""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import mass as M


def _qk(seed, B, H, N, D, spread=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, N, D)) * spread, rng.standard_normal((B, H, N, D)) * spread)


@pytest.mark.parametrize("N,block", [(150, 64), (128, 64), (70, 32), (5, 8)])
def test_rows_sum_to_query_count(N, block):
    """Every query's dense probabilities sum to one: a mass row sums to its block's query count."""
    q, k = _qk(N + block, 2, 2, N, 16, 2.0)
    m = M.block_mass(q, k, block, 0.25)
    nb = -(-N // block)
    counts = np.array([min(block, N - i * block) for i in range(nb)], float)
    np.testing.assert_allclose(m.sum(-1), np.broadcast_to(counts, m.shape[:-1]), rtol=0, atol=1e-11)
    assert (m >= 0).all()


def test_brute_force_tiny():
    """Loops over every (query, key) with math.exp, normalised per query."""
    q, k = _qk(5, 1, 1, 7, 4, 1.5)
    scale, block = 0.7, 3
    m = M.block_mass(q, k, block, scale)
    want = np.zeros((3, 3))
    for t in range(7):
        e = [math.exp(scale * sum(q[0, 0, t, d] * k[0, 0, c, d] for d in range(4))) for c in range(7)]
        z = sum(e)
        for c in range(7):
            want[t // block, c // block] += e[c] / z
    np.testing.assert_allclose(m[0, 0], want, rtol=1e-12, atol=1e-14)


def test_equal_keys_give_uniform_mass():
    """All keys equal: P = 1/N everywhere, so mass[i, j] = |block i| |block j| / N."""
    N, block = 100, 32
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, N, 8))
    k = np.broadcast_to(rng.standard_normal(8), (1, 1, N, 8)).copy()
    m = M.block_mass(q, k, block, 0.5)[0, 0]
    sizes = np.array([32, 32, 32, 4], float)
    np.testing.assert_allclose(m, np.outer(sizes, sizes) / N, rtol=1e-12)


def test_two_pass_form_matches():
    """mass = block sums of exp(scale q.k - LSE) with the dense LSE of the attention oracle:
    the form the two-pass kernel computes."""
    N, block, scale = 96, 32, 0.3
    q, k = _qk(11, 1, 2, N, 16, 2.0)
    v = np.zeros_like(q)
    _, lse = A.dense_attention(q, k, v, scale)
    m = M.block_mass(q, k, block, scale)
    for h in range(2):
        e = np.exp(scale * (q[0, h] @ k[0, h].T) - lse[0, h][:, None])
        np.testing.assert_allclose(m[0, h], e.reshape(3, 32, 3, 32).sum(axis=(1, 3)), rtol=1e-12)


def test_oracle_csr_hand_row():
    mass = np.array([[0.1, 0.5, 0.5, 0.05, 0.3]])
    assert M.oracle_csr(mass, [0, 3]).tolist() == [1, 2, 4]
    assert M.oracle_csr(mass, [0, 1]).tolist() == [1]          # tie 0.5/0.5 -> lower block
    assert M.oracle_csr(mass, [0, 0]).tolist() == []
    assert M.oracle_csr(mass, [0, 5]).tolist() == [0, 1, 2, 3, 4]


def test_oracle_keeps_the_most_mass():
    """For random rows and counts, no other choice of the same size keeps more mass."""
    rng = np.random.default_rng(7)
    nb, rows = 12, 40
    mass = rng.random((rows, nb))
    lens = rng.integers(0, nb + 1, rows)
    rp = np.concatenate([[0], np.cumsum(lens)])
    ci = M.oracle_csr(mass, rp)
    got = M.retained_mass(mass, rp, ci)
    for r in range(rows):
        cols = ci[rp[r]:rp[r + 1]]
        assert (np.diff(cols) > 0).all() and ((cols >= 0) & (cols < nb)).all()
        for _ in range(30):
            other = rng.choice(nb, lens[r], replace=False)
            assert got[r] >= mass[r, other].sum() - 1e-12
        assert math.isclose(got[r], np.sort(mass[r])[::-1][:lens[r]].sum(), rel_tol=1e-12, abs_tol=1e-15)


def test_full_csr_retains_everything():
    """A CSR listing every block keeps all the mass: each query's probability 1."""
    N, block = 90, 32
    q, k = _qk(2, 1, 1, N, 8)
    m = M.block_mass(q, k, block, 0.4)
    nb = 3
    rp = np.arange(nb + 1) * nb
    ci = np.tile(np.arange(nb), nb)
    np.testing.assert_allclose(M.retained_mass(m, rp, ci), [32, 32, 26], rtol=1e-12)
