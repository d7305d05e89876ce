"""GPU parity of residual compensation (bsa_residual, bsa_compensate and the anchor /
reuse sequence) against exact bf16 rounding and the fp64 oracle (oracle/residual.py)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import residual as OR
from parity import need_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [8, 1000, 1000003, 4 * 1024 * 1024])
def test_elementwise_bit_exact(n):
    """Each element formed in fp32 from the two bf16 inputs and rounded once (RNE): the
    same bits as the CPU doing the same; ragged tails of n % 8 elements included."""
    bsa = need_gpu()
    print(f"case n={n}", flush=True)
    g = torch.Generator("cpu").manual_seed(n)
    a = (torch.randn(n, generator=g) * 3).to(torch.bfloat16)
    b = (torch.randn(n, generator=g) * 3).to(torch.bfloat16)
    want_r = (a.float() - b.float()).to(torch.bfloat16)
    want_c = (a.float() + b.float()).to(torch.bfloat16)
    ad, bd = a.cuda(), b.cuda()
    r = bsa.residual(ad, bd)
    c = bsa.compensate(ad, bd)
    torch.cuda.synchronize()
    assert torch.equal(r.cpu().view(torch.int16), want_r.view(torch.int16))
    assert torch.equal(c.cpu().view(torch.int16), want_c.view(torch.int16))
    bsa.compensate(ad, bd, out=ad)            # the output may alias an input
    torch.cuda.synchronize()
    assert torch.equal(ad.cpu().view(torch.int16), want_c.view(torch.int16))


def test_misaligned_operand_is_rejected():
    bsa = need_gpu()
    a = torch.zeros(1025, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bsa.BsaError):
        bsa.residual(a[1:], a[:-1])


@pytest.mark.parametrize("block,D", [(64, 64), (128, 64)])
def test_anchor_reuse_matches_oracle(block, D):
    """Anchor at step 0 (dense output), reuse at steps 1, 2 with the anchor's CSR plus
    the cached residual: the oracle's outputs within the forward's tolerance, and
    closer to dense attention than the sparse output alone."""
    bsa = need_gpu()
    print(f"case block={block} D={D}", flush=True)
    B, H, N = 1, 2, 4 * block - 11
    nb = -(-N // block)
    steps = W.drifting_qkv(21, 3, 0.02, B, H, N, D, block)
    rng = np.random.default_rng(block + D)
    cols = [sorted({r % nb} | set(rng.choice(nb, 1).tolist())) for r in range(B * H * nb)]
    rp = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    ci = np.concatenate(cols).astype(np.int32)
    ref = OR.anchor_and_reuse(steps, rp, ci, block, 1.0 / np.sqrt(D))
    ar = bsa.AnchorReuse(block)
    for t, (q, k, v) in enumerate(steps):
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        o = ar.anchor(qd, kd, vd, rp, ci) if t == 0 else ar.reuse(qd, kd, vd)
        torch.cuda.synchronize()
        od, os_, oc = ref[t]
        got = o.float().cpu().numpy().astype(np.float64)
        err = np.abs(got - oc)
        print(f"step {t}: max abs {err.max():.3e} mean abs {err.mean():.3e}", flush=True)
        assert err.max() <= 3e-2 and err.mean() <= 3e-3
        if t > 0:
            assert np.linalg.norm(got - od) < 0.5 * np.linalg.norm(os_ - od)


def _rand_csr(rng, rows, nb, p):
    cols = []
    for r in range(rows):
        m = rng.random(nb) < p
        m[r % nb] = True
        cols.append(np.flatnonzero(m))
    rp = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    return rp, np.concatenate(cols).astype(np.int32)


@pytest.mark.parametrize("block,D,max_tiles", [(64, 64, 0), (64, 64, 2), (64, 128, 0),
                                               (64, 128, 2), (128, 64, 2), (128, 128, 0)])
def test_forward_compensated_matches_oracle(block, D, max_tiles):
    """bsa_forward_compensated: O = attention + R formed in fp32 and rounded once, for
    every kernel (64 x 64 and the general one) with and without cut rows (combined in
    the kernel or by the merge pass): the oracle's attention plus R within the forward's
    tolerance, the same LSE bits as bsa_forward, and with R = 0 the same O bits."""
    from oracle import attention as OA
    bsa = need_gpu()
    print(f"case block={block} D={D} max_tiles={max_tiles}", flush=True)
    B, H, N = 1, 3, 6 * block - 19
    nb = -(-N // block)
    rng = np.random.default_rng(block * 7 + D + max_tiles)
    rp, ci = _rand_csr(rng, B * H * nb, nb, 0.6)
    q, k, v = W.gaussian_qkv(500 + block + D, B, H, N, D)
    r = (torch.randn(B, H, N, D, generator=torch.Generator("cpu").manual_seed(9)) * 0.3
         ).to(torch.bfloat16)
    qd, kd, vd, rd = q.cuda(), k.cuda(), v.cuda(), r.cuda()
    work = bsa.Work.from_host(rp, D, block, max_tiles, "cuda", nb=nb, n_groups=2) \
        if max_tiles else None
    if work is not None:
        assert work.n_merges > 0
    o0, l0 = bsa.forward(qd, kd, vd, rp, ci, block, work=work)
    o1, l1 = bsa.forward(qd, kd, vd, rp, ci, block, work=work, residual=rd)
    oz, lz = bsa.forward(qd, kd, vd, rp, ci, block, work=work, residual=torch.zeros_like(rd))
    torch.cuda.synchronize()
    assert torch.equal(l0, l1) and torch.equal(l0, lz)
    assert torch.equal(o0, oz)
    O, _ = OA.block_sparse_attention(q, k, v, rp, ci, block, 1.0 / np.sqrt(D))
    want = O + r.float().numpy().astype(np.float64)
    err = np.abs(o1.float().cpu().numpy().astype(np.float64) - want)
    print(f"max abs {err.max():.3e} mean abs {err.mean():.3e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_forward_compensated_rejects_overlap():
    bsa = need_gpu()
    B, H, N, D, block = 1, 1, 128, 64, 64
    q = torch.zeros(B, H, N, D, dtype=torch.bfloat16, device="cuda")
    rp = np.array([0, 1, 2], np.int32)
    ci = np.array([0, 1], np.int32)
    out = torch.empty_like(q)
    with pytest.raises(bsa.BsaError):
        bsa.forward(q, q, q, rp, ci, block, out=out, residual=out)
