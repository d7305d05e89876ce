"""GPU parity of bsa_backward (dQ, dK, dV over the forward's CSR) against the fp64 backward
oracle (oracle/backward.py), through the C ABI; the forward's own O and LSE feed it."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import backward as OB
from parity import need_gpu

pytestmark = pytest.mark.gpu

# bf16 unit roundoff; P and dS are rounded to bf16 once as MFMA operands and every
# gradient once on output, O (for delta) is the forward's bf16 output.
U = 2.0 ** -9
MAX_REL = 8 * U      # max |err| over a tensor, relative to the tensor's max |ref|
MEAN_REL = U         # mean |err| over a tensor, relative to the tensor's max |ref|


def csr_from_cols(cols):
    rp = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    ci = (np.concatenate([np.asarray(c, np.int32) for c in cols]) if rp[-1]
          else np.zeros(0, np.int32)).astype(np.int32)
    return rp, ci


def run(bsa, q, k, v, do, rp, ci, block=64):
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = bsa.forward(qd, kd, vd, rp, ci, block)
    g = bsa.backward(qd, kd, vd, o, lse, dod, rp, ci, block)
    torch.cuda.synchronize()
    return [x.float().cpu().numpy().astype(np.float64) for x in g]


def compare(got, want, names=("dq", "dk", "dv")):
    for n, g, w in zip(names, got, want):
        assert np.isfinite(g).all(), n
        scale = max(np.abs(w).max(), 1e-30)
        err = np.abs(g - w)
        print(f"  {n}: max {err.max() / scale:.2e} mean {err.mean() / scale:.2e} (of max |ref|)",
              flush=True)
        assert err.max() <= MAX_REL * scale and err.mean() <= MEAN_REL * scale, n


@pytest.mark.parametrize("N,p,seed,D", [(512, 0.5, 0, 64), (245, 0.6, 1, 64), (64, 1.0, 2, 64),
                                        (1000, 0.3, 3, 64), (512, 0.5, 4, 128),
                                        (245, 0.6, 5, 128), (64, 1.0, 6, 128),
                                        (1000, 0.3, 7, 128)])
def test_backward_matches_oracle(N, p, seed, D):
    """Random CSR (diagonal kept), ragged last blocks, one row left empty; both head dims."""
    bsa = need_gpu()
    print(f"case N={N} p={p} D={D}", flush=True)
    B, H, block = 1, 2, 64
    nb = -(-N // block)
    q, k, v = W.gaussian_qkv(100 + seed, B, H, N, D)
    do = W.gaussian_qkv(200 + seed, B, H, N, D)[0]
    rng = np.random.default_rng(seed)
    cols = [sorted(set(np.flatnonzero(rng.random(nb) < p).tolist()) | {r % nb})
            for r in range(B * H * nb)]
    if nb > 1:
        cols[1] = []
    rp, ci = csr_from_cols(cols)
    got = run(bsa, q, k, v, do, rp, ci)
    want = OB.block_sparse_backward(q, k, v, rp, ci, block, 1 / np.sqrt(D), do)
    compare(got, want)
    if nb > 1:
        assert np.all(got[0][0, 0, 64:128] == 0.0)       # the empty row's dQ


@pytest.mark.parametrize("D", [64, 128])
def test_backward_unlisted_block_and_out_of_range_columns(D):
    """A key block no row lists gets dK = dV = 0; columns outside [0, nb) are ignored."""
    bsa = need_gpu()
    print(f"case D={D}", flush=True)
    B, H, N, block = 1, 1, 384, 64
    nb = N // block
    q, k, v = W.gaussian_qkv(5, B, H, N, D)
    do = W.gaussian_qkv(6, B, H, N, D)[0]
    cols = [[c for c in range(nb) if c != 3 and (c + r) % 2 == 0] or [0] for r in range(nb)]
    clean = csr_from_cols(cols)
    noisy = csr_from_cols([c + [-1, nb + 2] for c in cols])
    got = run(bsa, q, k, v, do, *noisy)
    want = OB.block_sparse_backward(q, k, v, *clean, block, 1 / np.sqrt(D), do)
    compare(got, want)
    assert np.all(got[1][0, 0, 192:256] == 0.0) and np.all(got[2][0, 0, 192:256] == 0.0)


@pytest.mark.parametrize("D", [64, 128])
def test_backward_dense_and_deterministic(D):
    """All-ones CSR (every key block listed by every row); two calls give the same bits."""
    bsa = need_gpu()
    B, H, N, block = 2, 2, 320, 64
    nb = N // block
    q, k, v = W.gaussian_qkv(9, B, H, N, D)
    do = W.gaussian_qkv(10, B, H, N, D)[0]
    rp, ci = csr_from_cols([list(range(nb))] * (B * H * nb))
    got = run(bsa, q, k, v, do, rp, ci)
    want = OB.block_sparse_backward(q, k, v, rp, ci, block, 1 / np.sqrt(D), do)
    compare(got, want)
    again = run(bsa, q, k, v, do, rp, ci)
    assert all(np.array_equal(a, b) for a, b in zip(got, again))


@pytest.mark.parametrize("N,H,D", [(2000, 2, 64), (4050, 1, 64), (2000, 1, 128)])
def test_backward_split_rows_and_columns(N, H, D):
    """Rows and key columns longer than the chunk length (twice the mean row length, at
    least 16) are cut into chunks whose fp32 partials are summed in chunk order: query
    block 0 lists every key block and every row lists key block 0 (2 and 4 chunks at
    nb = 32 and 64), the rest is the diagonal and its right neighbour; ragged N; a
    repeat call gives the same bits."""
    bsa = need_gpu()
    print(f"case N={N} H={H} D={D}", flush=True)
    B, block = 1, 64
    nb = -(-N // block)
    q, k, v = W.gaussian_qkv(300 + N, B, H, N, D)
    do = W.gaussian_qkv(400 + N, B, H, N, D)[0]
    cols = [list(range(nb)) if r % nb == 0 else sorted({0, r % nb, min(r % nb + 1, nb - 1)})
            for r in range(B * H * nb)]
    rp, ci = csr_from_cols(cols)
    got = run(bsa, q, k, v, do, rp, ci)
    want = OB.block_sparse_backward(q, k, v, rp, ci, block, 1 / np.sqrt(D), do)
    compare(got, want)
    again = run(bsa, q, k, v, do, rp, ci)
    assert all(np.array_equal(a, b) for a, b in zip(got, again))


@pytest.mark.parametrize("D", [64, 128])
def test_backward_twelve_heads_work_lists(D):
    """Twelve heads: one work list per die with one or two heads each, so workgroups
    whose list runs out take items from other lists; long rows and columns are split;
    ragged N.  Two calls give the same bits (an item's result does not depend on the
    workgroup that claims it)."""
    bsa = need_gpu()
    print(f"case D={D}", flush=True)
    B, H, N, block = 2, 6, 1500, 64
    nb = -(-N // block)
    q, k, v = W.gaussian_qkv(700 + D, B, H, N, D)
    do = W.gaussian_qkv(800 + D, B, H, N, D)[0]
    rng = np.random.default_rng(D)
    cols = []
    for r in range(B * H * nb):
        h, i = divmod(r, nb)
        dens = 0.9 if i < 2 else 0.15 * (1 + h % 3)
        cols.append(sorted(set(np.flatnonzero(rng.random(nb) < dens).tolist()) | {i, 0}))
    rp, ci = csr_from_cols(cols)
    got = run(bsa, q, k, v, do, rp, ci)
    want = OB.block_sparse_backward(q, k, v, rp, ci, block, 1 / np.sqrt(D), do)
    compare(got, want)
    again = run(bsa, q, k, v, do, rp, ci)
    assert all(np.array_equal(a, b) for a, b in zip(got, again))


@pytest.mark.parametrize("N,D", [(500, 64), (320, 64), (256, 128), (320, 128), (4000, 128)])
def test_backward_block128_matches_oracle(N, D):
    """Block 128 (refined to the 64-block CSR of the same mask): ragged N with and
    without a last 64-row half block (N % 128 of 116 and 64), uneven row lengths, one
    row left empty; the oracle works on the 128-block CSR directly."""
    bsa = need_gpu()
    print(f"case N={N} D={D}", flush=True)
    B, H, block = 1, 2, 128
    nb = -(-N // block)
    q, k, v = W.gaussian_qkv(700 + N + D, B, H, N, D)
    do = W.gaussian_qkv(800 + N + D, B, H, N, D)[0]
    rng = np.random.default_rng(N + D)
    cols = [sorted(set(rng.choice(nb, rng.integers(1, nb + 1), replace=False).tolist())
                   | {r % nb}) for r in range(B * H * nb)]
    if nb > 1:
        cols[1] = []
    rp, ci = csr_from_cols(cols)
    got = run(bsa, q, k, v, do, rp, ci, block)
    want = OB.block_sparse_backward(q, k, v, rp, ci, block, 1 / np.sqrt(D), do)
    compare(got, want)
    if nb > 1:
        assert np.all(got[0][0, 0, 128:256] == 0.0)      # the empty row's dQ
    again = run(bsa, q, k, v, do, rp, ci, block)
    assert all(np.array_equal(a, b) for a, b in zip(got, again))


def test_backward_dynamic_config_sampled_head():
    """The dynamic config's shape at D = 128 (B1 H16 N8192, block 64, 10 % top-k density
    built on the GPU); the oracle on one head."""
    bsa = need_gpu()
    w = W.make("dynamic")
    q, k, v = w.tensors()
    do = W.gaussian_qkv(w.seed + 2000, w.B, w.H, w.N, w.D)[0]
    qd, kd = q.cuda(), k.cuda()
    plan = bsa.Plan.create(w.B, w.H, w.N, w.D, w.block, w.density, w.prior(), w.budgets(),
                           w.force_diag, "cuda")
    rp_d, ci_d = bsa.build_mask(qd, kd, w.block, plan=plan)
    torch.cuda.synchronize()
    rp, ci = rp_d.cpu().numpy(), ci_d.cpu().numpy()
    got = run(bsa, q, k, v, do, rp, ci, w.block)
    nb = w.nb
    h = 5
    sub_rp = (rp[h * nb:(h + 1) * nb + 1] - rp[h * nb]).astype(np.int32)
    sub_ci = ci[rp[h * nb]:rp[(h + 1) * nb]]
    want = OB.block_sparse_backward(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], sub_rp, sub_ci,
                                    w.block, 1 / np.sqrt(w.D), do[:, h:h + 1])
    compare([g[:, h:h + 1] for g in got], want)


def test_backward_t2i_sampled_heads():
    """The t2i workload at full size (B2 H24 N4224, its static mask); the oracle on two
    heads (each head's gradients depend on that head only)."""
    bsa = need_gpu()
    w = W.make("t2i")
    q, k, v = w.tensors()
    do = W.gaussian_qkv(w.seed + 1000, w.B, w.H, w.N, w.D)[0]
    nb = w.nb
    prior = w.prior() | np.eye(nb, dtype=bool)
    rp, ci = csr_from_cols([np.flatnonzero(prior[r % nb]) for r in range(w.B * w.H * nb)])
    assert rp[nb] == 666
    got = run(bsa, q, k, v, do, rp, ci, w.block)
    for b, h in ((0, 0), (1, 23)):
        r0 = (b * w.H + h) * nb
        sub_rp = (rp[r0:r0 + nb + 1] - rp[r0]).astype(np.int32)
        sub_ci = ci[rp[r0]:rp[r0 + nb]]
        want = OB.block_sparse_backward(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                        v[b:b + 1, h:h + 1], sub_rp, sub_ci, w.block,
                                        1 / np.sqrt(w.D), do[b:b + 1, h:h + 1])
        compare([g[b:b + 1, h:h + 1] for g in got], want)


def test_backward_rejects_unsupported():
    bsa = need_gpu()
    q = torch.zeros((1, 1, 128, 96), dtype=torch.bfloat16, device="cuda")   # head dim 96
    lse = torch.zeros((1, 1, 128), dtype=torch.float32, device="cuda")
    rp = np.array([0, 1, 2], np.int32)
    ci = np.array([0, 1], np.int32)
    with pytest.raises(bsa.BsaError):
        bsa.backward(q, q, q, q, lse, q, rp, ci, 64)
