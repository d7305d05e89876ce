"""GPU parity of bsa_forward against the fp64 oracle, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from parity import compare_attention, need_gpu, token_rows

pytestmark = pytest.mark.gpu


def rand_csr(rng, B, H, nb, p, empty_rows=()):
    rows = []
    for r in range(B * H * nb):
        m = rng.random(nb) < p
        m[r % nb] = True
        if r in empty_rows:
            m[:] = False
        rows.append(np.flatnonzero(m))
    rp = np.concatenate([[0], np.cumsum([len(x) for x in rows])]).astype(np.int32)
    ci = np.concatenate(rows).astype(np.int32) if sum(len(x) for x in rows) else np.zeros(0, np.int32)
    return rp, ci


def run_and_compare(bsa, q, k, v, rp, ci, block, scale=None, work=None):
    B, H, N, D = q.shape
    dev = "cuda"
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = bsa.forward(qd, kd, vd, rp, ci, block, scale=scale, work=work)
    torch.cuda.synchronize()
    sc = scale if scale is not None else 1 / math.sqrt(D)
    O, L = OA.block_sparse_attention(q, k, v, rp, ci, block, sc)
    nb = -(-N // block)
    sel = token_rows(range(B * H * nb), nb, block, N, H)
    return compare_attention(o, lse, O, L, sel), o, lse


@pytest.mark.parametrize("block,D,N", [(64, 64, 500), (64, 128, 448), (128, 64, 200),
                                       (128, 128, 333), (64, 64, 64), (128, 128, 1)])
def test_small_ragged_all_shapes(block, D, N):
    """Several tiles, a ragged last block, every (block, D) the library supports."""
    bsa = need_gpu()
    print(f"case block={block} D={D} N={N}", flush=True)
    rng = np.random.default_rng(block + D + N)
    B, H = 2, 2
    q, k, v = W.gaussian_qkv(100 + N, B, H, N, D)
    nb = -(-N // block)
    rp, ci = rand_csr(rng, B, H, nb, 0.5)
    stats, _, _ = run_and_compare(bsa, q, k, v, rp, ci, block)
    print(stats)


def test_tiny_config_end_to_end():
    """Tiny workload: per-head Bernoulli prior + diagonal through the GPU builder, then forward."""
    bsa = need_gpu()
    w = W.make("tiny")
    q, k, v = w.tensors()
    from oracle import builder as OB
    rp_ref, ci_ref, _ = OB.build_mask(q, k, w.block, w.density, w.prior(), None, True)
    rp, ci = bsa.build_mask(q.cuda(), k.cuda(), w.block, w.density, w.prior(), None, True)
    assert np.array_equal(rp.cpu().numpy(), rp_ref)
    assert np.array_equal(ci.cpu().numpy()[:ci_ref.size], ci_ref)
    stats, _, _ = run_and_compare(bsa, q, k, v, rp.cpu().numpy(), ci.cpu().numpy(), w.block)
    print(stats)


def test_hand_case_gpu_sized():
    """q = e0, keys 0 / e0, values 0 / e0, scale ln 3: O[:,0] = 3/4 and LSE = ln 256 (or ln 64)."""
    bsa = need_gpu()
    N, D = 128, 64
    q = torch.zeros(1, 1, N, D, dtype=torch.bfloat16); q[..., 0] = 1
    k = torch.zeros_like(q); k[0, 0, 64:, 0] = 1
    v = torch.zeros_like(q); v[0, 0, 64:, 0] = 1
    o, lse = bsa.forward(q.cuda(), k.cuda(), v.cuda(), np.array([0, 2, 4]), np.array([0, 1, 0, 1]),
                         64, scale=math.log(3))
    o = o.float().cpu()[0, 0]; lse = lse.cpu()[0, 0]
    assert torch.allclose(o[:, 0], torch.full((N,), 0.75), atol=4e-3)
    assert o[:, 1:].abs().max() == 0
    assert torch.allclose(lse, torch.full((N,), math.log(256)), atol=1e-3)
    o, lse = bsa.forward(q.cuda(), k.cuda(), v.cuda(), np.array([0, 1, 3]), np.array([0, 0, 1]),
                         64, scale=math.log(3))
    o = o.float().cpu()[0, 0]; lse = lse.cpu()[0, 0]
    assert o[:64].abs().max() == 0
    assert torch.allclose(lse[:64], torch.full((64,), math.log(64)), atol=1e-3)


def test_empty_rows_and_explicit_scale():
    bsa = need_gpu()
    rng = np.random.default_rng(7)
    B, H, N, D, block = 1, 2, 300, 64, 64
    q, k, v = W.gaussian_qkv(7, B, H, N, D)
    nb = 5
    rp, ci = rand_csr(rng, B, H, nb, 0.4, empty_rows=(1, 7))
    stats, o, lse = run_and_compare(bsa, q, k, v, rp, ci, block, scale=0.3)
    assert (o[0, 0, 64:128].float() == 0).all()
    assert torch.isneginf(lse[0, 0, 64:128]).all()


def test_inactive_kv_perturbation_is_bit_identical():
    """Rows that do not list block j are bit-identical when block j's K/V change."""
    bsa = need_gpu()
    rng = np.random.default_rng(8)
    B, H, N, D, block = 1, 1, 512, 128, 64
    q, k, v = W.gaussian_qkv(8, B, H, N, D)
    nb = 8
    rp, ci = rand_csr(rng, B, H, nb, 0.4)
    j = 3
    o1, l1 = bsa.forward(q.cuda(), k.cuda(), v.cuda(), rp, ci, block)
    k2, v2 = k.clone(), v.clone()
    k2[..., j * block:(j + 1) * block, :] *= -3
    v2[..., j * block:(j + 1) * block, :] += 5
    o2, l2 = bsa.forward(q.cuda(), k2.cuda(), v2.cuda(), rp, ci, block)
    n_checked = 0
    for i in range(nb):
        if j not in ci[rp[i]:rp[i + 1]]:
            sl = slice(i * block, (i + 1) * block)
            assert torch.equal(o1[0, 0, sl], o2[0, 0, sl]) and torch.equal(l1[0, 0, sl], l2[0, 0, sl])
            n_checked += 1
    assert n_checked > 0


def test_launch_order_and_invalid_columns():
    """Results do not depend on the launch order; columns outside [0, nb) are skipped."""
    bsa = need_gpu()
    rng = np.random.default_rng(9)
    B, H, N, D, block = 2, 3, 700, 64, 64
    q, k, v = (t.cuda() for t in W.gaussian_qkv(9, B, H, N, D))
    nb = 11
    rp, ci = rand_csr(rng, B, H, nb, 0.3)
    o0, l0 = bsa.forward(q, k, v, rp, ci, block)
    w_host = bsa.Work.from_host(rp, D, block, 0, "cuda")
    o1, l1 = bsa.forward(q, k, v, rp, ci, block, work=w_host)
    w_dev = bsa.schedule(torch.from_numpy(rp).cuda(), nb)
    o2, l2 = bsa.forward(q, k, v, rp, ci, block, work=w_dev)
    assert torch.equal(o0, o1) and torch.equal(o0, o2) and torch.equal(l0, l1) and torch.equal(l0, l2)
    wk = w_dev.work.cpu().numpy()
    n = B * H * nb
    items = wk[:4 * n].reshape(-1, 4)
    assert wk[4 * n:].tolist() == [1, 0, n]                 # one group holding every item
    lens = np.diff(rp)
    assert sorted(items[:, 0].tolist()) == list(range(B * H * nb))
    assert np.array_equal(items[:, 1], rp[items[:, 0]]) and (items[:, 3] == -1).all()
    sizes = items[:, 2] - items[:, 1]
    assert np.array_equal(sizes, lens[items[:, 0]]) and (np.diff(sizes) <= 0).all()
    # insert junk columns (-1 and nb) at the front of every row
    rows = [np.concatenate([[-1, nb], ci[rp[r]:rp[r + 1]]]) for r in range(B * H * nb)]
    rp2 = np.concatenate([[0], np.cumsum([len(x) for x in rows])]).astype(np.int32)
    ci2 = np.concatenate(rows).astype(np.int32)
    o3, l3 = bsa.forward(q, k, v, rp2, ci2, block)
    assert torch.equal(o0, o3) and torch.equal(l0, l3)


@pytest.mark.parametrize("block,D,n_groups", [(64, 64, 8), (64, 64, 1), (64, 128, 8),
                                               (128, 64, 3)])
def test_item_queue_matches_static_order_and_resets(block, D, n_groups):
    """Items claimed from the per-group counters give the same bits as the static row
    order, call after call, and every call leaves the counters at zero.  The head count
    makes the item count exceed two static rounds of resident workgroups."""
    bsa = need_gpu()
    print(f"case block={block} D={D} n_groups={n_groups}", flush=True)
    rng = np.random.default_rng(block + D + n_groups)
    B, H, nb = 1, 48, 50
    N = nb * block - 5
    rp, ci = rand_csr(rng, B, H, nb, 0.12, empty_rows=(7, 300))
    work = bsa.Work.from_host(rp, D, block, 0, "cuda", nb=nb, n_groups=n_groups)
    assert work.n_items == B * H * nb
    for seed in (1, 2, 3):
        q, k, v = (t.cuda() for t in W.gaussian_qkv(300 + seed, B, H, N, D))
        o0, l0 = bsa.forward(q, k, v, rp, ci, block)
        o1, l1 = bsa.forward(q, k, v, rp, ci, block, work=work)
        torch.cuda.synchronize()
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
        assert int(work.workspace[:64 * 4096].count_nonzero()) == 0


@pytest.mark.parametrize("block,D,max_tiles,n_groups", [(64, 64, 2, 8), (64, 64, 3, 1),
                                                         (64, 64, 1, 8), (64, 128, 2, 8),
                                                         (64, 128, 1, 1)])
def test_cut_rows_repeat_bitwise_and_counters_reset(block, D, max_tiles, n_groups):
    """Cut rows combined once their last chunk is stored: the oracle's values, the same
    bits call after call, and every item and merge counter back at zero after each call.
    Enough items that most of them are claimed from the per-group counters."""
    bsa = need_gpu()
    print(f"case block={block} D={D} max_tiles={max_tiles} n_groups={n_groups}", flush=True)
    rng = np.random.default_rng(7 * block + D + max_tiles + n_groups)
    B, H, nb = 1, 16, 20
    N = nb * block - 9
    rp, ci = rand_csr(rng, B, H, nb, 0.5, empty_rows=(3, 100))
    work = bsa.Work.from_host(rp, D, block, max_tiles, "cuda", nb=nb, n_groups=n_groups)
    assert work.n_merges > 0
    n_cnt = bsa.forward_workspace_bytes(work.n_slots, D, block) - work.n_slots * block * (D + 2) * 4
    assert n_cnt >= 64 * 4096 + 8 * work.n_slots
    q, k, v = W.gaussian_qkv(400 + max_tiles, B, H, N, D)
    stats, o0, l0 = run_and_compare(bsa, q, k, v, rp, ci, block, work=work)
    print(stats)
    assert int(work.workspace[:n_cnt].count_nonzero()) == 0
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for _ in range(2):
        o1, l1 = bsa.forward(qd, kd, vd, rp, ci, block, work=work)
        torch.cuda.synchronize()
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
        assert int(work.workspace[:n_cnt].count_nonzero()) == 0


@pytest.mark.parametrize("block,D,max_tiles", [(64, 64, 1), (64, 64, 3), (64, 128, 1),
                                               (64, 128, 2), (64, 128, 3), (128, 64, 4),
                                               (128, 128, 1)])
def test_cut_rows_match_oracle(block, D, max_tiles):
    """Rows cut into chunks (partials in the workspace, then combined) against the oracle."""
    bsa = need_gpu()
    print(f"case block={block} D={D} max_tiles={max_tiles}", flush=True)
    rng = np.random.default_rng(block + D + max_tiles)
    B, H, N = 1, 3, 9 * block - 17
    q, k, v = W.gaussian_qkv(200 + max_tiles, B, H, N, D)
    nb = 9
    rp, ci = rand_csr(rng, B, H, nb, 0.6, empty_rows=(4,))
    ci = ci.copy()
    ci[rp[5]:rp[6]] = ci[rp[5]:rp[6]][::-1].copy()     # any column order is allowed
    work = bsa.Work.from_host(rp, D, block, max_tiles, "cuda")
    assert work.n_merges > 0
    stats, o, lse = run_and_compare(bsa, q, k, v, rp, ci, block, work=work)
    print(stats)
    assert (o[0, 0, 4 * block:5 * block].float() == 0).all()       # CSR row 4 is empty
    assert torch.isneginf(lse[0, 0, 4 * block:5 * block]).all()


def test_no_lse_output():
    bsa = need_gpu()
    q, k, v = (t.cuda() for t in W.gaussian_qkv(11, 1, 1, 256, 64))
    rp = np.array([0, 1, 3, 4, 8], np.int32); ci = np.array([0, 0, 1, 2, 0, 1, 2, 3], np.int32)
    o1, l1 = bsa.forward(q, k, v, rp, ci, 64)
    o2, l2 = bsa.forward(q, k, v, rp, ci, 64, return_lse=False)
    assert l2 is None and torch.equal(o1, o2)


def test_all_ones_equals_dense_oracle():
    """BSA-DiT §4.3: check the block-sparse kernel against dense attention first."""
    bsa = need_gpu()
    B, H, N, D, block = 1, 2, 640, 128, 128
    q, k, v = W.gaussian_qkv(12, B, H, N, D)
    nb = 5
    rp = (np.arange(B * H * nb + 1) * nb).astype(np.int32)
    ci = np.tile(np.arange(nb), B * H * nb).astype(np.int32)
    o, lse = bsa.forward(q.cuda(), k.cuda(), v.cuda(), rp, ci, block)
    O, L = OA.dense_attention(q, k, v, 1 / math.sqrt(D))
    sel = token_rows(range(B * H * nb), nb, block, N, H)
    print(compare_attention(o, lse, O, L, sel))


def test_graph_replay_matches_eager():
    """The t2i forward (work list with cut rows combined in the kernel) captured in a HIP
    graph: every replay, with eager launches and synchronisations between the replays,
    gives the eager result bit for bit, and the claim and merge counters keep working."""
    bsa = need_gpu()
    w = W.make("t2i")
    q, k, v = w.tensors()
    dev = "cuda"
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    plan = bsa.Plan.create(w.B, w.H, w.N, w.D, w.block, w.density, w.prior(), w.budgets(),
                           w.force_diag, dev)
    ci = torch.empty(max(plan.nnz, 1), dtype=torch.int32, device=dev)
    bsa.build_mask(qd, kd, w.block, plan=plan, col_idx=ci)
    o_ref, l_ref = bsa.forward(qd, kd, vd, plan.row_ptr, ci, w.block, work=plan)
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bsa.forward(qd, kd, vd, plan.row_ptr, ci, w.block, work=plan, out=o, lse=lse)
    for rep in range(4):
        o.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), rep
        o2, l2 = bsa.forward(qd, kd, vd, plan.row_ptr, ci, w.block, work=plan)
        torch.cuda.synchronize()
        assert torch.equal(o2, o_ref) and torch.equal(l2, l_ref), rep
