"""Pins for the mask-builder oracle: hand cases, brute force, closed forms, invariants."""
import itertools
import math

import numpy as np
import pytest

from conftest import load_golden
from oracle import builder as Bd


def block_constant(vecs, block, N):
    """[1,1,N,D] tensor whose block i is filled with vecs[i]."""
    vecs = np.asarray(vecs, float)
    x = np.empty((1, 1, N, vecs.shape[1]))
    for t in range(N):
        x[0, 0, t] = vecs[t // block]
    return x


@pytest.mark.parametrize("N", [8, 7])
def test_hand_block_constant(N):
    """(B1) block-constant integer inputs: pooled means, scores and selections by hand."""
    g = load_golden("builder_hand.json")
    q = block_constant(g["qv"], 2, N)
    k = block_constant(g["kv"], 2, N)
    pq, pk = Bd.mean_pool(q, 2), Bd.mean_pool(k, 2)
    assert np.array_equal(pq[0, 0], np.array(g["qv"], float))
    assert np.array_equal(pk[0, 0], np.array(g["kv"], float))
    assert np.array_equal(Bd.block_scores(pq, pk)[0, 0], np.array(g["scores"], float))
    for c in g["cases"]:
        assert Bd.budget(4, c["density"]) == c["K"]
        rp, ci, gaps = Bd.build_mask(q, k, 2, c["density"], None, None, c["force_diag"])
        rows = [ci[rp[r]:rp[r + 1]].tolist() for r in range(4)]
        assert rows == c["rows"]
        assert gaps.tolist() == c["gaps"]


def test_partial_block_mean_uses_valid_tokens():
    x = np.zeros((1, 1, 5, 1)); x[0, 0, :, 0] = [1, 2, 3, 4, 10]
    p = Bd.mean_pool(x, 4)
    assert p[0, 0, :, 0].tolist() == [2.5, 10.0]


@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_subsets(seed):
    """(B2) the fill is the max-sum subset of the non-prior columns (distinct scores)."""
    rng = np.random.default_rng(seed)
    nb = 7
    s = rng.permutation(nb).astype(float) + rng.random(nb) * 0.1
    sel = rng.random(nb) < 0.3
    for K in range(nb + 1):
        cols, gap = Bd.select_row(s, sel, K)
        fill = max(0, K - int(sel.sum()))
        cand = [j for j in range(nb) if not sel[j]]
        best = max(itertools.combinations(cand, fill), key=lambda c: sum(s[list(c)]))
        expect = sorted(set(np.flatnonzero(sel).tolist()) | set(best))
        assert cols.tolist() == expect
        if 0 < fill < len(cand):
            left = [j for j in cand if j not in best]
            assert math.isclose(gap, min(s[list(best)]) - max(s[left]))
        else:
            assert gap == math.inf


def test_bruteforce_ties_prefer_lower_index():
    """(B2) with ties, among max-sum subsets the lexicographically smallest is chosen."""
    s = np.array([1.0, 2.0, 1.0, 2.0, 0.0, 1.0])
    sel = np.zeros(6, dtype=bool)
    for K in range(7):
        cols, _ = Bd.select_row(s, sel, K)
        best = max(itertools.combinations(range(6), K),
                   key=lambda c: (sum(s[list(c)]), [-j for j in c]))
        assert cols.tolist() == sorted(best)


def test_density_table():
    """(B3) density -> blocks per row, round half up, at least one."""
    table = {(128, 0.10): 13, (256, 0.10): 26, (250, 0.05): 13, (66, 0.15): 10,
             (8, 1.0): 8, (8, 0.0): 0, (8, 0.01): 1, (64, 0.1): 6, (4, 0.5): 2}
    for (nb, d), K in table.items():
        assert Bd.budget(nb, d) == K, (nb, d)


def test_density_one_gives_all_ones():
    rng = np.random.default_rng(11)
    q, k = rng.standard_normal((2, 1, 2, 40, 4))
    rp, ci, _ = Bd.build_mask(q, k, 8, 1.0)
    nb = 5
    assert np.array_equal(rp, np.arange(2 * nb + 1) * nb)
    assert np.array_equal(ci, np.tile(np.arange(nb), 2 * nb))


@pytest.mark.parametrize("seed", range(3))
def test_invariants(seed):
    """(B4) counts, prior inclusion, score ordering, ascending unique columns."""
    rng = np.random.default_rng(seed)
    B, H, N, D, block = 1, 3, 150, 8, 10
    nb = 15
    q, k = rng.standard_normal((2, B, H, N, D))
    prior = (rng.random((nb, nb)) < 0.15).astype(np.uint8)
    budgets = rng.integers(0, nb + 1, nb)
    rp, ci, gaps = Bd.build_mask(q, k, block, 0.0, prior, budgets, True)
    S = Bd.block_scores(Bd.mean_pool(q, block), Bd.mean_pool(k, block))
    counts = Bd.plan_counts(B, H, nb, 0.0, prior, budgets, True)
    assert np.array_equal(np.diff(rp), counts)
    for h in range(H):
        for i in range(nb):
            r = h * nb + i
            cols = ci[rp[r]:rp[r + 1]]
            sel = prior[i].astype(bool).copy(); sel[i] = True
            assert (np.diff(cols) > 0).all() and cols.min() >= 0 and cols.max() < nb
            assert set(np.flatnonzero(sel)) <= set(cols.tolist())
            assert len(cols) == max(sel.sum(), budgets[i])
            filled = [j for j in cols if not sel[j]]
            out = [j for j in range(nb) if j not in set(cols.tolist())]
            if filled and out:
                assert min(S[0, h, i, filled]) >= max(S[0, h, i, out])
                assert math.isclose(gaps[r], min(S[0, h, i, filled]) - max(S[0, h, i, out]))


def test_per_head_prior():
    """A 4-D prior is read per (b, h)."""
    prior = np.zeros((1, 2, 3, 3), dtype=np.uint8)
    prior[0, 1, 0, 2] = 1
    q = np.zeros((1, 2, 9, 2))
    rp, ci, _ = Bd.build_mask(q, q, 3, 0.0, prior, None, True)
    assert ci[rp[0]:rp[1]].tolist() == [0]
    assert ci[rp[3]:rp[4]].tolist() == [0, 2]
