"""Pins of the token-level selection oracle (CPU): eigenvectors, exact partitions,
mass conservation, and reductions to the dense and block-sparse attention oracles
(oracle/tokensel.py, from the page on the quality gap of sparse attention in diffusion
transformers, section on token-level selection with tile-aligned query groups)."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import mass as M
from oracle import tokensel as T
from conftest import load_golden


def test_principal_direction_is_the_top_eigenvector():
    rng = np.random.default_rng(1)
    D = 16
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    x = rng.standard_normal((300, 1)) * 6.0 @ u[None, :] + rng.standard_normal((300, D)) * 0.5
    v = T.principal_direction(x, iters=30)
    w, e = np.linalg.eigh(np.cov(x.T))
    assert abs(v @ e[:, -1]) > 0.9999 and abs(v @ u) > 0.99


def test_partition_is_exact_and_tile_sized():
    rng = np.random.default_rng(2)
    C = 16
    for g in (1, 2, 3, 5, 8):
        x = rng.standard_normal((g * C, 8))
        groups = T.median_split_groups(x, C)
        assert groups.shape == (g, C)
        assert sorted(groups.ravel().tolist()) == list(range(g * C))
        assert all((np.diff(r) > 0).all() for r in groups)


def test_separated_clusters_are_recovered():
    """Four far-apart clusters of C tokens, interleaved in token order: each group is one
    cluster, in the order of the two cuts (median along the top direction, then within)."""
    rng = np.random.default_rng(3)
    C, D = 8, 6
    centres = np.array([[-30.0, 5, 0, 0, 0, 0], [-30.0, -5, 0, 0, 0, 0],
                        [30.0, 5, 0, 0, 0, 0], [30.0, -5, 0, 0, 0, 0]])
    lab = np.tile(np.arange(4), C)
    x = centres[lab] + rng.standard_normal((4 * C, D)) * 0.1
    groups = T.median_split_groups(x, C)
    found = [set(lab[g].tolist()) for g in groups]
    assert all(len(f) == 1 for f in found)
    assert sorted(f.pop() for f in found) == [0, 1, 2, 3]


def test_odd_group_count_cuts_at_a_tile_boundary():
    """Three groups: the first cut keeps C on the low side of the top direction."""
    rng = np.random.default_rng(4)
    C = 8
    x = rng.standard_normal((3 * C, 5)) * 0.1
    x[:, 0] += np.repeat([-10.0, 0.0, 10.0], C)[rng.permutation(3 * C)]
    groups = T.median_split_groups(x, C)
    means = [x[g, 0].mean() for g in groups]
    assert max(abs(m) for m in means) > 9.0
    assert all(np.ptp(x[g, 0]) < 2.0 for g in groups)     # each group one band


def test_token_mass_conservation_and_block_sums():
    """A group's token masses sum to its size; for groups that are whole query blocks, the
    token masses summed over key blocks are the block mass of oracle/mass.py."""
    rng = np.random.default_rng(5)
    N, D, C = 96, 8, 32
    q, k = rng.standard_normal((N, D)), rng.standard_normal((N, D))
    groups = np.arange(N).reshape(N // C, C)
    tm = T.token_mass(q, k, groups, 0.4)
    np.testing.assert_allclose(tm.sum(1), C, rtol=1e-12)
    bm = M.block_mass(q[None, None], k[None, None], C, 0.4)[0, 0]
    np.testing.assert_allclose(tm.reshape(3, 3, C).sum(-1), bm, rtol=1e-12)


def test_select_tokens_hand():
    m = np.array([[0.2, 0.9, 0.2, 0.5, 0.9]])
    assert T.select_tokens(m, 2).tolist() == [[1, 4]]
    assert T.select_tokens(m, 3).tolist() == [[1, 3, 4]]
    assert T.select_tokens(m, 4).tolist() == [[0, 1, 3, 4]]     # tie 0.2/0.2 -> token 0


def test_gathered_attention_reduces_to_dense_and_block_sparse():
    rng = np.random.default_rng(6)
    N, D, C = 64, 8, 16
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    groups = T.median_split_groups(q, C)
    O, L = T.gathered_attention(q, k, v, groups, np.tile(np.arange(N), (N // C, 1)), 0.3)
    Od, Ld = A.masked_attention(q, k, v, np.ones((N, N), bool), 0.3)
    np.testing.assert_allclose(O, Od, atol=1e-12)
    np.testing.assert_allclose(L, Ld, atol=1e-12)
    # contiguous groups and whole-block token lists: the block-sparse oracle
    gb = np.arange(N).reshape(N // C, C)
    cols = [[0, 2], [1], [1, 3], [0, 1, 2, 3]]
    toks = [np.concatenate([np.arange(c * C, c * C + C) for c in cs]) for cs in cols]
    rp = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    ci = np.concatenate(cols).astype(np.int32)
    Ob, Lb = A.block_sparse_attention(q[None, None], k[None, None], v[None, None], rp, ci, C, 0.3)
    for g, t in zip(gb, toks):
        o, l = T.gathered_attention(q, k, v, g[None], t[None], 0.3)
        np.testing.assert_allclose(o[g], Ob[0, 0, g], atol=1e-12)
        np.testing.assert_allclose(l[g], Lb[0, 0, g], atol=1e-12)


def test_power_iteration_hand_golden():
    """tests/golden/query_groups_hand.json (worked by hand): 2-D points in +/- pairs whose
    scatter matrix is diag(490, 392); from u = (1, 1.5) the direction after k steps has
    tan = 1.5 * 0.8^k, and the single median split depends on k being 8 and on the start."""
    g = load_golden("query_groups_hand.json")
    half = np.array(g["half_points"], dtype=np.float64)
    x = np.empty((2 * len(half), 2))
    x[0::2], x[1::2] = half, -half
    v = T.principal_direction(x)
    assert abs(v[1] / v[0] - g["tan_theta_after_8"]) < 1e-12
    assert T.median_split_groups(x, g["C"]).tolist() == g["groups"]
