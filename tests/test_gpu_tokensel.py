"""GPU parity of the token-level selection steps (query groups, token mass, top-k tokens)
against the fp64 oracle (oracle/tokensel.py), through the C ABI."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import tokensel as OT
from parity import LSE_ABS, O_MAX_ABS, O_MEAN_ABS, need_gpu

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
                                   (8, 64, 64), (6, 128, 64), (40, 64, 128), (66, 64, 64)])
def test_query_groups_recover_separated_clusters(G, C, D):
    """Far-apart clusters leave no near-tie at any cut: the GPU groups are the oracle's.
    The two largest cases split segments above 1024 tokens, whose scatter matrices come
    from 512-token slice partials."""
    bsa = need_gpu()
    print(f"case G={G} C={C} D={D}", flush=True)
    q = clustered_q(G * 10 + D, G, C, D)
    groups = bsa.query_groups(q.cuda(), C)
    torch.cuda.synchronize()
    got = groups.cpu().numpy()
    for h in range(q.shape[1]):
        want = OT.median_split_groups(q[0, h].float().numpy(), C)
        assert np.array_equal(got[0, h], want)


# Per-split tolerance on projections (relative to the segment's largest |projection|).
# The GPU forms the scatter matrix in fp32 from bf16 hi/lo products (relative error near
# 2^-16 per product), runs the eight power-iteration steps and the projections in fp32;
# through eight steps that moves the direction by well under 1e-4 relative, so projections
# of the GPU and of the fp64 oracle differ by less than 1e-3 of the largest one.
SPLIT_EPS = 1e-3


def check_splits(x, groups, C, eps_rel=SPLIT_EPS):
    """Walk the GPU's split tree (groups numbered depth first, first part first): for every
    segment of g > 1 groups, project its tokens on the oracle's fp64 principal direction of
    that segment; every token the GPU put left must project at most eps above every token it
    put right, and where the oracle's cut has a gap above 2 eps the two cuts are the same.
    Returns (splits checked exactly, splits within the tolerance only)."""
    exact = loose = 0

    def rec(s, g):
        nonlocal exact, loose
        if g == 1:
            return
        toks = np.concatenate(groups[s:s + g])
        sub = x[toks]
        p = (sub - sub.mean(0)) @ OT.principal_direction(sub)
        gl = g // 2
        nl = gl * C
        left = np.isin(toks, np.concatenate(groups[s:s + gl]))
        eps = eps_rel * np.abs(p).max()
        assert p[left].max() <= p[~left].min() + eps, (s, g, p[left].max(), p[~left].min())
        ps = np.sort(p)
        if ps[nl] - ps[nl - 1] > 2 * eps:
            assert np.array_equal(np.sort(toks[np.lexsort((toks, p))[:nl]]), np.sort(toks[left]))
            exact += 1
        else:
            loose += 1
        rec(s, gl)
        rec(s + gl, g - gl)

    rec(0, len(groups))
    return exact, loose


@pytest.mark.parametrize("N,C,D,H", [(4224, 64, 64, 2), (2048, 128, 128, 1), (8192, 64, 128, 1)])
def test_query_groups_random_split_by_split(N, C, D, H):
    """Random queries at full head lengths (t2i, and lengths whose top segments are split
    from 512-token slice partials): a partition into tile-sized ascending groups, checked
    split by split against the oracle's fp64 direction of the same segment (see
    check_splits); exact wherever the median has a gap above the fp32 tolerance."""
    bsa = need_gpu()
    print(f"case N={N} C={C} D={D}", flush=True)
    q, _, _ = W.gaussian_qkv(77 + N, 1, H, N, D)
    groups = bsa.query_groups(q.cuda(), C)
    torch.cuda.synchronize()
    got = groups.cpu().numpy()
    for h in range(H):
        x = q[0, h].float().numpy().astype(np.float64)
        g = got[0, h]
        assert sorted(g.ravel().tolist()) == list(range(N))
        assert all((np.diff(r) > 0).all() for r in g)
        exact, loose = check_splits(x, g, C)
        print(f"head {h}: {exact} splits exact, {loose} within tolerance", flush=True)
        assert exact + loose == N // C - 1


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


def random_lists(seed, G, N, T):
    """Per group, T distinct tokens of [0, N) in random order (the order is free)."""
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(N, T, replace=False) for _ in range(G)]).astype(np.int32)


def run_gather(bsa, q, k, v, groups, tokens, out=None):
    o, lse = bsa.gather_forward(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(groups).cuda(),
                                torch.from_numpy(tokens).cuda(), out=out)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check_rows(o, lse, O, L, rows):
    err = np.abs(o[rows] - O[rows])
    print(f"  o max {err.max():.3e} mean {err.mean():.3e}", flush=True)
    assert err.max() <= O_MAX_ABS and err.mean() <= O_MEAN_ABS
    fin = np.isfinite(L[rows])
    assert np.array_equal(np.isfinite(lse[rows]), fin)
    if fin.any():
        assert np.abs(lse[rows][fin] - L[rows][fin]).max() <= LSE_ABS


@pytest.mark.parametrize("N,T,D", [(512, 100, 64), (512, 64, 64), (1024, 1, 64), (1024, 33, 64),
                                   (1024, 640, 64), (320, 320, 64), (512, 100, 128),
                                   (512, 64, 128), (1024, 1, 128), (1024, 33, 128),
                                   (1024, 640, 128), (320, 320, 128)])
def test_gather_forward_matches_oracle(N, T, D):
    """Oracle groups (median split) and seeded token lists: ragged last tiles, a tile half
    with no key, one token, every token; both head dims."""
    bsa = need_gpu()
    print(f"case N={N} T={T} D={D}", flush=True)
    B, H = 1, 2
    q, k, v = W.gaussian_qkv(N + T + D, B, H, N, D)
    G = N // 64
    groups = np.stack([OT.median_split_groups(q[0, h].float().numpy(), 64) for h in range(H)])
    tokens = np.stack([random_lists(7 * h + T, G, N, T) for h in range(H)])
    o, lse = run_gather(bsa, q, k, v, groups[None].astype(np.int32), tokens[None])
    for h in range(H):
        O, L = OT.gathered_attention(q[0, h], k[0, h], v[0, h], groups[h], tokens[h],
                                     1 / np.sqrt(D))
        check_rows(o[0, h], lse[0, h], O, L, np.arange(N))


def test_gather_forward_d128_long_head_sampled():
    """A dynamic-config head at D = 128 (N = 8192, 128 groups, 820 tokens each, about
    10 %); the oracle on every thirteenth group."""
    bsa = need_gpu()
    B, H, N, D, T = 1, 2, 8192, 128, 820
    q, k, v = W.gaussian_qkv(8192 + 128, B, H, N, D)
    G = N // 64
    rng = np.random.default_rng(6)
    groups = np.stack([rng.permutation(N).reshape(G, 64) for _ in range(H)]).astype(np.int32)
    groups.sort(axis=-1)
    tokens = np.stack([random_lists(11 + h, G, N, T) for h in range(H)])
    o, lse = run_gather(bsa, q, k, v, groups[None], tokens[None])
    for h in range(H):
        for g in range(0, G, 13):
            O, L = OT.gathered_attention(q[0, h], k[0, h], v[0, h], groups[h, g:g + 1],
                                         tokens[h, g:g + 1], 1 / np.sqrt(D))
            check_rows(o[0, h], lse[0, h], O, L, groups[h, g])


def test_gather_forward_t2i_head_length_sampled():
    """A full t2i head (N = 4224, 66 groups, 640 tokens each, about 15 %); the oracle on
    every eleventh group."""
    bsa = need_gpu()
    B, H, N, D, T = 1, 2, 4224, 64, 640
    q, k, v = W.gaussian_qkv(4224, B, H, N, D)
    G = N // 64
    rng = np.random.default_rng(5)
    groups = np.stack([rng.permutation(N).reshape(G, 64) for _ in range(H)]).astype(np.int32)
    groups.sort(axis=-1)
    tokens = np.stack([random_lists(h, G, N, T) for h in range(H)])
    o, lse = run_gather(bsa, q, k, v, groups[None], tokens[None])
    for h in range(H):
        for g in range(0, G, 11):
            O, L = OT.gathered_attention(q[0, h], k[0, h], v[0, h], groups[h, g:g + 1],
                                         tokens[h, g:g + 1], 1 / 8.0)
            check_rows(o[0, h], lse[0, h], O, L, groups[h, g])


@pytest.mark.parametrize("D", [64, 128])
def test_gather_forward_skips_out_of_range_entries(D):
    """Token entries outside [0, N) are skipped; so are group slots outside [0, N)."""
    bsa = need_gpu()
    B, H, N, T = 1, 1, 256, 90
    q, k, v = W.gaussian_qkv(31, B, H, N, D)
    G = N // 64
    groups = np.arange(N, dtype=np.int32).reshape(G, 64)
    tokens = random_lists(3, G, N, T)
    bad_t = tokens.copy()
    bad_t[:, ::7] = -1
    bad_t[:, 3::11] = N + 5
    bad_g = groups.copy()
    bad_g[1, 5] = -3
    out = torch.full((B, H, N, D), 3.0, dtype=torch.bfloat16, device="cuda")
    o, lse = run_gather(bsa, q, k, v, bad_g[None, None], bad_t[None, None], out=out)
    for g in range(G):
        keep = bad_t[g][(bad_t[g] >= 0) & (bad_t[g] < N)]
        O, L = OT.gathered_attention(q[0, 0], k[0, 0], v[0, 0], groups[g:g + 1], keep[None],
                                     1 / np.sqrt(D))
        rows = bad_g[g][bad_g[g] >= 0]
        check_rows(o[0, 0], lse[0, 0], O, L, rows)
    assert (o[0, 0, 64 + 5] == 3.0).all() and np.isneginf(lse[0, 0, 64 + 5])


@pytest.mark.parametrize("D", [64, 128])
def test_gather_forward_empty_lists_and_unnamed_rows(D):
    """T = 0: every named row gets O = 0 and LSE = -inf; rows no group names keep `out`."""
    bsa = need_gpu()
    B, H, N = 1, 2, 384
    q, k, v = W.gaussian_qkv(8, B, H, N, D)
    groups = np.arange(128, dtype=np.int32).reshape(1, 1, 2, 64).repeat(H, 1)
    out = torch.full((B, H, N, D), -2.0, dtype=torch.bfloat16, device="cuda")
    o, lse = run_gather(bsa, q, k, v, groups, np.zeros((1, H, 2, 0), np.int32), out=out)
    assert (o[:, :, :128] == 0).all() and np.isneginf(lse[:, :, :128]).all()
    assert (o[:, :, 128:] == -2.0).all() and np.isneginf(lse[:, :, 128:]).all()
    # a few tokens, the same unnamed rows
    tokens = np.stack([random_lists(h, 2, N, 5) for h in range(H)])[None]
    o, lse = run_gather(bsa, q, k, v, groups, tokens, out=out)
    assert (o[:, :, 128:] == -2.0).all()
    for h in range(H):
        O, L = OT.gathered_attention(q[0, h], k[0, h], v[0, h], groups[0, h], tokens[0, h],
                                     1 / np.sqrt(D))
        check_rows(o[0, h], lse[0, h], O, L, np.arange(128))


def test_gather_forward_rejects_unsupported():
    bsa = need_gpu()
    q = torch.zeros((1, 1, 128, 96), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((1, 1, 2, 64), dtype=torch.int32, device="cuda")
    t = torch.zeros((1, 1, 2, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(bsa.BsaError):
        bsa.gather_forward(q, q, q, g, t)        # head dim 96 is not supported
    q64 = torch.zeros((1, 1, 128, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        bsa.gather_forward(q64, q64, q64, g[..., :32].contiguous(), t)


def test_token_mass_t2i_sampled_heads():
    """The t2i workload at full size (B2 H24 N4224 D64, 66 groups of 64 per head, the
    launch that splits each group's keys into two slices), seeded random groups, the LSE
    of the dense forward; the oracle on two heads (a head's masses depend on that head
    only), and every group's masses sum to its query count."""
    bsa = need_gpu()
    w = W.make("t2i")
    q, k, _ = w.tensors()
    qd, kd = q.cuda(), k.cuda()
    B, H, N, C = w.B, w.H, w.N, 64
    G = N // C
    rng = np.random.default_rng(4224)
    groups = np.stack([np.sort(rng.permutation(N).reshape(G, C), axis=-1)
                       for _ in range(B * H)]).reshape(B, H, G, C).astype(np.int32)
    lse = dense_lse(bsa, qd, kd, 64)
    mass = bsa.token_mass(qd, kd, lse, torch.from_numpy(groups).cuda())
    torch.cuda.synchronize()
    got = mass.cpu().numpy().astype(np.float64)
    for b, h in ((0, 3), (1, 20)):
        want = OT.token_mass(q[b, h], k[b, h], groups[b, h], 1.0 / np.sqrt(w.D))
        err = np.abs(got[b, h] - want)
        print(f"head ({b},{h}): max abs {err.max():.3e}", flush=True)
        assert np.all(err <= 2e-4 * want + 1e-6), err.max()
    np.testing.assert_allclose(got.sum(-1), C, rtol=2e-4)
