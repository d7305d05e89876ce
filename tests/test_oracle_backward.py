"""Pins of the backward oracle (oracle/backward.py): central finite differences of the
forward oracle, torch float64 autograd through scaled_dot_product_attention (dense and with
the equivalent token mask), and closed forms of the softmax gradient."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import backward as BW


def random_csr(rng, n_rows, nb, p=0.5, allow_empty=False):
    cols = []
    for r in range(n_rows):
        c = np.flatnonzero(rng.random(nb) < p)
        if c.size == 0 and not allow_empty:
            c = np.array([r % nb])
        cols.append(c)
    rp = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    ci = (np.concatenate(cols) if rp[-1] else np.zeros(0)).astype(np.int32)
    return rp, ci


def token_mask(rp, ci, N, block, r0, nb):
    """Boolean [N, N] token mask of the CSR rows r0 .. r0 + nb - 1 (one head)."""
    m = np.zeros((N, N), bool)
    for i in range(nb):
        for c in ci[rp[r0 + i]:rp[r0 + i + 1]]:
            m[i * block:(i + 1) * block, c * block:(c + 1) * block] = True
    return m


def test_finite_differences():
    """Every input element: the oracle's gradient of L = sum dO * O equals the central
    difference of the forward oracle (ragged last block, one empty CSR row)."""
    rng = np.random.default_rng(11)
    B, H, N, D, block = 1, 2, 10, 3, 4
    nb = 3
    q, k, v, do = (rng.standard_normal((B, H, N, D)) for _ in range(4))
    rp, ci = random_csr(rng, B * H * nb, nb, 0.6)
    # make row 4 (head 1, block 1) empty
    cols = [list(ci[rp[r]:rp[r + 1]]) for r in range(B * H * nb)]
    cols[4] = []
    rp = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    ci = np.array([c for cs in cols for c in cs], np.int32)
    scale = 0.7
    dq, dk, dv = BW.block_sparse_backward(q, k, v, rp, ci, block, scale, do)

    def loss(q_, k_, v_):
        O, _ = A.block_sparse_attention(q_, k_, v_, rp, ci, block, scale)
        return float((do * O).sum())

    eps = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v, name: xp}
            args_m = {"q": q, "k": k, "v": v, name: xm}
            num[idx] = (loss(**{a + "_": b for a, b in args_p.items()}) -
                        loss(**{a + "_": b for a, b in args_m.items()})) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=1e-7, err_msg=name)
    assert np.all(dq[0, 1, 4:8] == 0.0)          # the empty row


def _torch_grads(q, k, v, do, scale, mask=None):
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    am = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=am, scale=scale)
    o.backward(torch.from_numpy(do))
    return [x.grad.numpy() for x in t]


@pytest.mark.parametrize("N,block", [(100, 32), (64, 16)])
def test_dense_equals_torch_autograd(N, block):
    rng = np.random.default_rng(N)
    B, H, D = 1, 2, 16
    q, k, v, do = (rng.standard_normal((B, H, N, D)) for _ in range(4))
    nb = -(-N // block)
    rp = (np.arange(B * H * nb + 1) * nb).astype(np.int32)
    ci = np.tile(np.arange(nb, dtype=np.int32), B * H * nb)
    got = BW.block_sparse_backward(q, k, v, rp, ci, block, 0.25, do)
    want = _torch_grads(q, k, v, do, 0.25)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, atol=1e-10)


def test_sparse_equals_torch_autograd_with_token_mask():
    rng = np.random.default_rng(5)
    B, H, N, D, block = 1, 2, 96, 8, 16
    nb = N // block
    q, k, v, do = (rng.standard_normal((B, H, N, D)) for _ in range(4))
    rp, ci = random_csr(rng, B * H * nb, nb, 0.4)
    got = BW.block_sparse_backward(q, k, v, rp, ci, block, 0.3, do)
    for h in range(H):
        m = token_mask(rp, ci, N, block, h * nb, nb)
        want = _torch_grads(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], do[:, h:h + 1], 0.3, m)
        for g, w in zip(got, want):
            np.testing.assert_allclose(g[:, h:h + 1], w, atol=1e-10)


def test_closed_forms():
    """Per head: the rows of dK sum to 0 (a shared shift of the keys moves every score of
    a row by the same amount); the rows of dV sum to the dO rows that see a key; keys that
    no row lists get exactly 0; a constant V gives dQ = dK = 0; dO = 0 gives 0."""
    rng = np.random.default_rng(8)
    B, H, N, D, block = 2, 1, 80, 5, 16
    nb = N // block
    q, k, v, do = (rng.standard_normal((B, H, N, D)) for _ in range(4))
    rp, ci = random_csr(rng, B * H * nb, nb, 0.5, allow_empty=True)
    # block 2 is listed by no row
    cols = [[c for c in ci[rp[r]:rp[r + 1]] if c != 2] for r in range(B * H * nb)]
    cols[0] = []                                           # and row 0 is empty
    rp = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    ci = np.array([c for cs in cols for c in cs], np.int32)
    dq, dk, dv = BW.block_sparse_backward(q, k, v, rp, ci, block, 0.5, do)
    seen = np.zeros((B, H, N), bool)
    for r in range(B * H * nb):
        bh, i = divmod(r, nb)
        if rp[r + 1] > rp[r]:
            seen[bh // H, bh % H, i * block:(i + 1) * block] = True
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-11)
    np.testing.assert_allclose(dv.sum(axis=2), (do * seen[..., None]).sum(axis=2), atol=1e-11)
    assert np.all(dk[:, :, 32:48] == 0.0) and np.all(dv[:, :, 32:48] == 0.0)
    vc = np.broadcast_to(rng.standard_normal(D), v.shape).copy()
    dq2, dk2, _ = BW.block_sparse_backward(q, k, vc, rp, ci, block, 0.5, do)
    np.testing.assert_allclose(dq2, 0.0, atol=1e-12)
    np.testing.assert_allclose(dk2, 0.0, atol=1e-12)
    z = BW.block_sparse_backward(q, k, v, rp, ci, block, 0.5, np.zeros_like(do))
    assert all(np.all(x == 0.0) for x in z)
