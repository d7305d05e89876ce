"""GPU parity of the exact block mass, the equal-density block oracle and the retained
mass of a CSR against the fp64 oracle (oracle/mass.py), through the C ABI."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import mass as OM
from parity import need_gpu

pytestmark = pytest.mark.gpu


def rand_csr(rng, rows, nb, p):
    lens = []
    cols = []
    for r in range(rows):
        m = rng.random(nb) < p
        cols.append(np.flatnonzero(m))
        lens.append(len(cols[-1]))
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ci = np.concatenate(cols).astype(np.int32) if sum(lens) else np.zeros(0, np.int32)
    return rp, ci


def dense_lse(bsa, q, k, block):
    B, H, N, D = q.shape
    nb = -(-N // block)
    rows = B * H * nb
    rp = (np.arange(rows + 1) * nb).astype(np.int32)
    ci = np.tile(np.arange(nb, dtype=np.int32), rows)
    _, lse = bsa.forward(q, k, k, rp, ci, block)
    return lse


@pytest.mark.parametrize("block,D,N", [(64, 64, 300), (64, 128, 200), (128, 64, 333),
                                       (128, 128, 130), (64, 64, 64), (128, 64, 1)])
def test_block_mass_matches_oracle(block, D, N):
    """Several blocks, a ragged last block, every (block, D) the library supports."""
    bsa = need_gpu()
    print(f"case block={block} D={D} N={N}", flush=True)
    q, k, _ = W.gaussian_qkv(500 + N, 1, 2, N, D)
    qd, kd = q.cuda(), k.cuda()
    lse = dense_lse(bsa, qd, kd, block)
    mass = bsa.block_mass(qd, kd, lse, block)
    torch.cuda.synchronize()
    ref = OM.block_mass(q, k, block, 1.0 / np.sqrt(D))
    got = mass.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    print(f"max abs {err.max():.3e}, max rel {(err / np.maximum(ref, 1e-6)).max():.3e}", flush=True)
    assert np.all(err <= 1e-4 * ref + 2e-6)
    nb = -(-N // block)
    counts = np.array([min(block, N - i * block) for i in range(nb)], float)
    np.testing.assert_allclose(got.sum(-1), np.broadcast_to(counts, got.shape[:-1]), rtol=2e-4)


@pytest.mark.parametrize("nb,p", [(9, 0.4), (66, 0.15), (130, 0.3), (300, 0.05)])
def test_select_by_mass_is_the_top_of_each_row(nb, p):
    """The GPU picks, per row, the same blocks as the oracle deciding on the same fp32
    masses (ties to the lower block), including rows with no block and full rows."""
    bsa = need_gpu()
    print(f"case nb={nb} p={p}", flush=True)
    rng = np.random.default_rng(nb)
    rows = 3 * nb
    mass = rng.random((rows, nb)).astype(np.float32)
    mass[1, :] = 0.5                        # all tied: lowest blocks win
    mass[2, :] = np.repeat(rng.random((nb + 1) // 2), 2)[:nb].astype(np.float32)  # tied pairs
    rp, _ = rand_csr(rng, rows, nb, p)
    lens = np.diff(rp)
    lens[0] = 0
    lens[3] = nb
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ci = bsa.select_by_mass(torch.from_numpy(mass).cuda(), rp)
    torch.cuda.synchronize()
    want = OM.oracle_csr(mass.astype(np.float64), rp)
    assert np.array_equal(ci.cpu().numpy(), want)


def test_select_by_mass_reports_rows_longer_than_nb():
    bsa = need_gpu()
    mass = torch.rand((4, 5), device="cuda")
    rp = np.array([0, 2, 8, 9, 10], np.int32)     # row 1 asks for 6 of 5 blocks
    with pytest.raises(bsa.BsaError):
        bsa.select_by_mass(mass, rp)


def test_csr_mass_matches_oracle():
    bsa = need_gpu()
    rng = np.random.default_rng(3)
    rows, nb = 200, 40
    mass = (rng.random((rows, nb)) * 3).astype(np.float32)
    rp, ci = rand_csr(rng, rows, nb, 0.3)
    out = bsa.csr_mass(torch.from_numpy(mass).cuda(), rp, ci)
    torch.cuda.synchronize()
    want = OM.retained_mass(mass.astype(np.float64), rp, ci)
    np.testing.assert_allclose(out.cpu().numpy(), want, rtol=1e-5, atol=1e-6)


def test_block_oracle_keeps_at_least_the_mean_pool_mass():
    """End to end on a small dynamic-mask workload: the two-pass block oracle at the
    mean-pool CSR's density keeps, row by row, at least the mass the mean-pool top-k
    keeps, and as much as the fp64 oracle's own choice (up to rounding)."""
    bsa = need_gpu()
    w = W.make("tiny")
    q, k, _ = w.tensors()
    qd, kd = q.cuda(), k.cuda()
    rp, ci = bsa.build_mask(qd, kd, w.block, w.density, w.prior(), None, True)
    ci_o, mass = bsa.block_oracle(qd, kd, rp, w.block)
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy()
    ref = OM.block_mass(q, k, w.block, 1.0 / np.sqrt(w.D))
    kept_pool = OM.retained_mass(ref, rp_h, ci.cpu().numpy())
    kept_gpu = OM.retained_mass(ref, rp_h, ci_o.cpu().numpy())
    kept_best = OM.retained_mass(ref, rp_h, OM.oracle_csr(ref, rp_h))
    print(f"mean kept: mean-pool {kept_pool.mean():.3f}, oracle {kept_gpu.mean():.3f}", flush=True)
    assert np.all(kept_gpu >= kept_pool - 1e-4 * w.block)
    assert np.all(kept_gpu >= kept_best - 1e-4 * w.block)
    got = bsa.csr_mass(mass, rp, ci_o).cpu().numpy()
    np.testing.assert_allclose(got, kept_gpu, rtol=2e-4, atol=1e-5)


def test_block_mass_t2i_sampled_heads():
    """The t2i workload at full size (B2 H24 N4224 D64, block 64), as the benchmark runs
    it: the dense LSE from the forward over the all-ones CSR, then the block masses of
    every head on the GPU; the oracle on two heads (a head's masses depend on that head
    only), and every row sums to its block's query count."""
    bsa = need_gpu()
    w = W.make("t2i")
    q, k, _ = w.tensors()
    qd, kd = q.cuda(), k.cuda()
    lse = dense_lse(bsa, qd, kd, w.block)
    mass = bsa.block_mass(qd, kd, lse, w.block)
    torch.cuda.synchronize()
    got = mass.cpu().numpy().astype(np.float64)
    for b, h in ((0, 3), (1, 20)):
        ref = OM.block_mass(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], w.block,
                            1.0 / np.sqrt(w.D))[0, 0]
        err = np.abs(got[b, h] - ref)
        print(f"head ({b},{h}): max abs {err.max():.3e}", flush=True)
        assert np.all(err <= 1e-4 * ref + 2e-6)
    np.testing.assert_allclose(got.sum(-1), float(w.block), rtol=2e-4)
