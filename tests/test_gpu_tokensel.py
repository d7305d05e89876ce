"""GPU parity of the token-level selection steps (query groups, token mass, top-k tokens)
against the fp64 oracle (oracle/tokensel.py), through the C ABI."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import tokensel as OT
from parity import need_gpu

pytestmark = pytest.mark.gpu


def clustered_q(seed, G, C, D, H=2):
    """G far-apart clusters of C queries each, interleaved in token order."""
    rng = np.random.default_rng(seed)
    out = []
    for h in range(H):
        centres = rng.standard_normal((G, D)) * 20.0
        lab = rng.permutation(np.repeat(np.arange(G), C))
        out.append(centres[lab] + rng.standard_normal((G * C, D)) * 0.3)
    return torch.from_numpy(np.stack(out)[None].astype(np.float32)).to(torch.bfloat16)


def dense_lse(bsa, q, k, block):
    B, H, N, D = q.shape
    nb = -(-N // block)
    rows = B * H * nb
    rp = (np.arange(rows + 1) * nb).astype(np.int32)
    ci = np.tile(np.arange(nb, dtype=np.int32), rows)
    _, lse = bsa.forward(q, k, k, rp, ci, block)
    return lse


@pytest.mark.parametrize("G,C,D", [(1, 64, 64), (2, 64, 64), (3, 64, 64), (5, 64, 128),
                                   (8, 64, 64), (6, 128, 64)])
def test_query_groups_recover_separated_clusters(G, C, D):
    """Far-apart clusters leave no near-tie at any cut: the GPU groups are the oracle's."""
    bsa = need_gpu()
    print(f"case G={G} C={C} D={D}", flush=True)
    q = clustered_q(G * 10 + D, G, C, D)
    groups = bsa.query_groups(q.cuda(), C)
    torch.cuda.synchronize()
    got = groups.cpu().numpy()
    for h in range(q.shape[1]):
        want = OT.median_split_groups(q[0, h].float().numpy(), C)
        assert np.array_equal(got[0, h], want)


def test_query_groups_random_are_valid_and_as_tight():
    """Random queries of a full t2i head length: a partition into tile-sized ascending
    groups whose within-group scatter matches the oracle's to 1 % (cuts near the median
    may go either way in fp32)."""
    bsa = need_gpu()
    N, C, D = 4224, 64, 64
    q, _, _ = W.gaussian_qkv(77, 1, 2, N, D)
    groups = bsa.query_groups(q.cuda(), C)
    torch.cuda.synchronize()
    got = groups.cpu().numpy()
    for h in range(2):
        x = q[0, h].float().numpy().astype(np.float64)
        g = got[0, h]
        assert sorted(g.ravel().tolist()) == list(range(N))
        assert all((np.diff(r) > 0).all() for r in g)
        want = OT.median_split_groups(x, C)
        scat = lambda gs: sum(((x[r] - x[r].mean(0)) ** 2).sum() for r in gs)
        print(f"head {h}: scatter gpu {scat(g):.1f} oracle {scat(want):.1f}", flush=True)
        assert abs(scat(g) - scat(want)) <= 0.01 * scat(want)


@pytest.mark.parametrize("C,D,N", [(64, 64, 1024), (64, 128, 512), (128, 64, 768)])
def test_token_mass_matches_oracle(C, D, N):
    bsa = need_gpu()
    print(f"case C={C} D={D} N={N}", flush=True)
    q, k, _ = W.gaussian_qkv(900 + N, 1, 2, N, D)
    qd, kd = q.cuda(), k.cuda()
    groups = bsa.query_groups(qd, C)
    lse = dense_lse(bsa, qd, kd, 64)
    mass = bsa.token_mass(qd, kd, lse, groups)
    torch.cuda.synchronize()
    got = mass.cpu().numpy().astype(np.float64)
    g = groups.cpu().numpy()
    for h in range(2):
        want = OT.token_mass(q[0, h], k[0, h], g[0, h], 1.0 / np.sqrt(D))
        err = np.abs(got[0, h] - want)
        assert np.all(err <= 2e-4 * want + 1e-6), err.max()
        np.testing.assert_allclose(got[0, h].sum(-1), C, rtol=2e-4)


@pytest.mark.parametrize("N,k", [(1024, 154), (4224, 640), (300, 300), (64, 1)])
def test_select_tokens_matches_oracle(N, k):
    """Top-k tokens per row, decided on the same fp32 masses: the oracle's lists exactly
    (rows with tied masses included)."""
    bsa = need_gpu()
    print(f"case N={N} k={k}", flush=True)
    rng = np.random.default_rng(N + k)
    m = rng.random((6, N)).astype(np.float32)
    m[1] = 0.25
    m[2] = np.repeat(rng.random((N + 1) // 2), 2)[:N]
    toks = bsa.select_tokens(torch.from_numpy(m).cuda(), k)
    torch.cuda.synchronize()
    assert np.array_equal(toks.cpu().numpy(), OT.select_tokens(m.astype(np.float64), k))
