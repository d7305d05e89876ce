"""Pins for the attention oracle: library routine, closed forms, invariants.

BSA-DiT §4.3 asks that a block-sparse kernel first be checked against dense
attention; these tests check the oracle itself that way and more.
"""
import math

import numpy as np
import pytest
import torch

from conftest import load_golden, parse_num
from oracle import attention as A


def rand_csr(rng, B, H, nb, p, force_diag=True, allow_empty=False):
    rows = []
    for r in range(B * H * nb):
        i = r % nb
        m = rng.random(nb) < p
        if force_diag:
            m[i] = True
        if not allow_empty and not m.any():
            m[rng.integers(nb)] = True
        rows.append(np.flatnonzero(m))
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum([len(x) for x in rows])
    return row_ptr, (np.concatenate(rows) if rows else np.zeros(0, np.int64))


def full_csr(B, H, nb):
    row_ptr = np.arange(B * H * nb + 1, dtype=np.int64) * nb
    col_idx = np.tile(np.arange(nb), B * H * nb)
    return row_ptr, col_idx


def token_mask(row_ptr, col_idx, b, h, H, nb, block, N):
    """Independent expansion of a CSR to a boolean [N, N] token mask."""
    m = np.zeros((N, N), dtype=bool)
    for i in range(nb):
        r = (b * H + h) * nb + i
        for j in col_idx[row_ptr[r]:row_ptr[r + 1]]:
            m[i * block:(i + 1) * block, j * block:(j + 1) * block] = True
    return m


@pytest.mark.parametrize("N,block", [(96, 32), (100, 32), (7, 4)])
def test_all_ones_equals_torch_sdpa(N, block):
    """(O1) all blocks active == textbook attention (torch SDPA, float64)."""
    rng = np.random.default_rng(1)
    B, H, D = 2, 3, 16
    q, k, v = (rng.standard_normal((B, H, N, D)) for _ in range(3))
    scale = 0.37
    nb = -(-N // block)
    rp, ci = full_csr(B, H, nb)
    O, L = A.block_sparse_attention(q, k, v, rp, ci, block, scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).numpy()
    lse = torch.logsumexp(scale * tq @ tk.transpose(-1, -2), dim=-1).numpy()
    assert np.abs(O - ref).max() < 1e-12
    assert np.abs(L - lse).max() < 1e-12
    O2, L2 = A.dense_attention(q, k, v, scale)
    assert np.abs(O2 - ref).max() < 1e-12 and np.abs(L2 - lse).max() < 1e-12


@pytest.mark.parametrize("N,block", [(128, 16), (77, 16)])
def test_sparse_equals_torch_sdpa_with_token_mask(N, block):
    """Block CSR == SDPA with the equivalent boolean token mask; LSE == torch.logsumexp."""
    rng = np.random.default_rng(2)
    B, H, D = 1, 2, 8
    q, k, v = (rng.standard_normal((B, H, N, D)) for _ in range(3))
    nb = -(-N // block)
    rp, ci = rand_csr(rng, B, H, nb, 0.4)
    scale = 1 / math.sqrt(D)
    O, L = A.block_sparse_attention(q, k, v, rp, ci, block, scale)
    for b in range(B):
        for h in range(H):
            m = torch.from_numpy(token_mask(rp, ci, b, h, H, nb, block, N))
            tq, tk, tv = (torch.from_numpy(x[b, h]) for x in (q, k, v))
            ref = torch.nn.functional.scaled_dot_product_attention(
                tq[None], tk[None], tv[None], attn_mask=m[None], scale=scale)[0].numpy()
            s = (scale * tq @ tk.T).masked_fill(~m, float("-inf"))
            lse = torch.logsumexp(s, dim=-1).numpy()
            assert np.abs(O[b, h] - ref).max() < 1e-12
            assert np.abs(L[b, h] - lse).max() < 1e-12


def test_q_zero_closed_form():
    """(O2) Q = 0: every active key weighs the same, O = mean of active V, LSE = ln(#keys)."""
    rng = np.random.default_rng(3)
    B, H, N, D, block = 1, 2, 90, 4, 16
    nb = -(-N // block)
    q = np.zeros((B, H, N, D))
    k, v = rng.standard_normal((2, B, H, N, D))
    rp, ci = rand_csr(rng, B, H, nb, 0.5)
    O, L = A.block_sparse_attention(q, k, v, rp, ci, block, 0.5)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                r = (b * H + h) * nb + i
                keys = np.concatenate([np.arange(j * block, min(N, (j + 1) * block))
                                       for j in sorted(ci[rp[r]:rp[r + 1]])])
                rows = slice(i * block, min(N, (i + 1) * block))
                assert np.allclose(O[b, h, rows], v[b, h, keys].mean(0), atol=1e-13)
                assert np.allclose(L[b, h, rows], math.log(len(keys)), atol=1e-13)


def test_v_constant():
    """(O3) V = c everywhere => O = c whatever the mask."""
    rng = np.random.default_rng(4)
    B, H, N, D, block = 1, 1, 70, 5, 8
    nb = -(-N // block)
    q, k = rng.standard_normal((2, B, H, N, D))
    v = np.full((B, H, N, D), -1.25)
    rp, ci = rand_csr(rng, B, H, nb, 0.3)
    O, _ = A.block_sparse_attention(q, k, v, rp, ci, block, 0.9)
    assert np.abs(O + 1.25).max() < 1e-14


def test_hand_two_token():
    """(O4) hand-worked case from tests/golden/attention_hand.json."""
    g = load_golden("attention_hand.json")["two_token"]
    q = np.array(g["q"], float)[None, None]
    k = np.array(g["k"], float)[None, None]
    v = np.array(g["v"], float)[None, None]
    for c in g["cases"]:
        O, L = A.block_sparse_attention(q, k, v, c["row_ptr"], c["col_idx"], g["block"], math.log(3))
        assert np.allclose(O[0, 0], np.array(c["O"]), atol=1e-15)
        assert np.allclose(L[0, 0], [parse_num(x) for x in c["LSE"]], atol=1e-15)


def gpu_sized_inputs():
    N, D = 128, 64
    q = np.zeros((1, 1, N, D)); q[..., 0] = 1.0
    k = np.zeros((1, 1, N, D)); k[0, 0, 64:, 0] = 1.0
    v = np.zeros((1, 1, N, D)); v[0, 0, 64:, 0] = 1.0
    return q, k, v


def test_hand_gpu_sized():
    """(O4) the same construction at D = 64, block = 64, N = 128."""
    g = load_golden("attention_hand.json")["gpu_sized"]
    q, k, v = gpu_sized_inputs()
    c0, c1 = g["cases"]
    rp, ci = np.array([0, 2, 4]), np.array([0, 1, 0, 1])
    O, L = A.block_sparse_attention(q, k, v, rp, ci, 64, math.log(3))
    assert np.allclose(O[0, 0, :, 0], c0["O_col0"], atol=1e-14)
    assert np.abs(O[0, 0, :, 1:]).max() == c0["O_other"]
    assert np.allclose(L, parse_num(c0["LSE"]), atol=1e-13)
    rp, ci = np.array([0, 1, 3]), np.array([0, 0, 1])
    O, L = A.block_sparse_attention(q, k, v, rp, ci, 64, math.log(3))
    assert np.abs(O[0, 0, :64]).max() == c1["O_col0_rows_block0"]
    assert np.allclose(L[0, 0, :64], parse_num(c1["LSE_rows_block0"]), atol=1e-13)
    assert np.allclose(O[0, 0, 64:, 0], 0.75, atol=1e-14)


def test_inactive_perturbation_and_order():
    """(O5) K/V of inactive blocks do not matter; the order of a row's columns does not matter."""
    rng = np.random.default_rng(5)
    B, H, N, D, block = 1, 1, 64, 4, 8
    nb = N // block
    q, k, v = rng.standard_normal((3, B, H, N, D))
    # row 0 sees blocks {0, 5}; every other row sees only its diagonal
    ci = np.array([5, 0] + list(range(1, nb)))
    rp = np.concatenate([[0, 2], 2 + np.arange(1, nb)])
    O, L = A.block_sparse_attention(q, k, v, rp, ci, block, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, 3 * block:4 * block] += 100.0  # block 3 is inactive for row 0
    v2[0, 0, 3 * block:4 * block] -= 7.0
    O2, L2 = A.block_sparse_attention(q, k2, v2, rp, ci, block, 0.5)
    assert np.array_equal(O[0, 0, :block], O2[0, 0, :block])
    assert np.array_equal(L[0, 0, :block], L2[0, 0, :block])
    ci_sorted = np.array([0, 5] + list(range(1, nb)))
    O3, L3 = A.block_sparse_attention(q, k, v, rp, ci_sorted, block, 0.5)
    assert np.array_equal(O, O3) and np.array_equal(L, L3)


def test_indicator_of_inactive_block_gives_zero_column():
    """(O5) V column = indicator of block j: O column is exactly 0 on rows where j is inactive."""
    rng = np.random.default_rng(6)
    B, H, N, D, block = 1, 1, 48, 3, 8
    nb = N // block
    q, k, v = rng.standard_normal((3, B, H, N, D))
    v[..., 1] = 0.0
    v[0, 0, 2 * block:3 * block, 1] = 1.0
    rp, ci = rand_csr(rng, B, H, nb, 0.5)
    O, _ = A.block_sparse_attention(q, k, v, rp, ci, block, 0.7)
    for i in range(nb):
        act = set(ci[rp[i]:rp[i + 1]].tolist())
        col = O[0, 0, i * block:(i + 1) * block, 1]
        if 2 in act:
            assert (col > 0).all()
        else:
            assert (col == 0).all()


def test_block_diagonal_is_per_block_dense():
    """(O5) diagonal-only mask == independent dense attention inside every block (SDPA)."""
    rng = np.random.default_rng(7)
    B, H, N, D, block = 1, 2, 40, 6, 8
    nb = N // block
    q, k, v = rng.standard_normal((3, B, H, N, D))
    rp = np.arange(B * H * nb + 1)
    ci = np.tile(np.arange(nb), B * H)
    O, _ = A.block_sparse_attention(q, k, v, rp, ci, block, 0.4)
    for i in range(nb):
        sl = slice(i * block, (i + 1) * block)
        tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x[:, :, sl])) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.4).numpy()
        assert np.abs(O[:, :, sl] - ref).max() < 1e-12


def test_rows_sum_to_one_and_lse_bounds():
    """(O5) softmax rows sum to 1 (V = 1 gives O = 1); max score <= LSE <= max + ln(#keys)."""
    rng = np.random.default_rng(8)
    B, H, N, D, block = 1, 1, 60, 4, 8
    nb = -(-N // block)
    q, k = rng.standard_normal((2, B, H, N, D)) * 3
    v = np.ones((B, H, N, D))
    rp, ci = rand_csr(rng, B, H, nb, 0.4)
    O, L = A.block_sparse_attention(q, k, v, rp, ci, block, 0.5)
    assert np.abs(O - 1).max() < 1e-13
    for i in range(nb):
        keys = np.concatenate([np.arange(j * block, min(N, (j + 1) * block)) for j in ci[rp[i]:rp[i + 1]]])
        for a in range(i * block, min(N, (i + 1) * block)):
            s = 0.5 * k[0, 0, keys] @ q[0, 0, a]
            assert s.max() - 1e-12 <= L[0, 0, a] <= s.max() + math.log(len(keys)) + 1e-12


def test_empty_row():
    """Reading: a row with no active block has O = 0 and LSE = -inf."""
    rng = np.random.default_rng(9)
    q, k, v = rng.standard_normal((3, 1, 1, 16, 2))
    rp = np.array([0, 0, 2])
    ci = np.array([0, 1])
    O, L = A.block_sparse_attention(q, k, v, rp, ci, 8, 1.0)
    assert (O[0, 0, :8] == 0).all() and np.isneginf(L[0, 0, :8]).all()
    assert np.isfinite(O[0, 0, 8:]).all()


def test_rows_subset_matches_full():
    rng = np.random.default_rng(10)
    q, k, v = rng.standard_normal((3, 1, 2, 50, 4))
    nb = 7
    rp, ci = rand_csr(rng, 1, 2, nb, 0.5)
    O, L = A.block_sparse_attention(q, k, v, rp, ci, 8, 0.3)
    O2, L2 = A.block_sparse_attention(q, k, v, rp, ci, 8, 0.3, rows=[3, 9])
    assert np.array_equal(O2[0, 0, 24:32], O[0, 0, 24:32])
    assert np.array_equal(L2[0, 1, 16:24], L[0, 1, 16:24])
    assert np.isnan(O2[0, 0, 0]).all()
