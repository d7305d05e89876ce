"""bsa_forward_noalloc (the forward whose work-list workspace is the library's static
device array) against bsa_forward with a caller workspace, through the C ABI: the same
kernels run, so the outputs must agree bit for bit.  Two calls in a row, the second on a
smaller input, then a repeat of the first (the array keeps the previous call's contents,
and every call clears its counters itself)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from parity import need_gpu

pytestmark = pytest.mark.gpu

BSA_ERR_CAPACITY = -4


def rand_csr(rng, B, H, nb, p):
    rows = []
    for r in range(B * H * nb):
        m = rng.random(nb) < p
        m[r % nb] = True
        rows.append(np.flatnonzero(m))
    rp = np.concatenate([[0], np.cumsum([len(x) for x in rows])]).astype(np.int32)
    return rp, np.concatenate(rows).astype(np.int32)


def call_noalloc(bsa, q, k, v, rp, ci, block, work, out, lse):
    B, H, N, D = q.shape
    vp = ctypes.c_void_p
    st = bsa.lib.bsa_forward_noalloc(
        vp(q.data_ptr()), vp(k.data_ptr()), vp(v.data_ptr()), B, H, N, D, block,
        vp(rp.data_ptr()), vp(ci.data_ptr()), vp(work.work.data_ptr()), work.n_items,
        work.n_merges, work.n_slots, -1.0, vp(out.data_ptr()), vp(lse.data_ptr()),
        vp(torch.cuda.current_stream().cuda_stream))
    return st


def case_t2i(bsa):
    w = W.make("t2i")
    q, k, v = (t.cuda() for t in w.tensors())
    plan = bsa.Plan.create(w.B, w.H, w.N, w.D, w.block, w.density, w.prior(), w.budgets(),
                           w.force_diag, "cuda")
    rp, ci = bsa.build_mask(q, k, w.block, plan=plan)
    return q, k, v, rp, ci, w.block, plan.work


def case_small(bsa):
    # head dim 128 (the general kernel and the merge kernel), rows cut into chunks
    rng = np.random.default_rng(5)
    B, H, block, D = 1, 3, 64, 128
    nb = 9
    N = nb * block - 21
    rp, ci = rand_csr(rng, B, H, nb, 0.6)
    work = bsa.Work.from_host(rp, D, block, 2, "cuda", nb=nb, n_groups=2)
    assert work.n_merges > 0
    q, k, v = (t.cuda() for t in W.gaussian_qkv(77, B, H, N, D))
    return (q, k, v, torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(), block, work)


def check(bsa, case):
    q, k, v, rp, ci, block, work = case
    print(f"case B{q.shape[0]} H{q.shape[1]} N{q.shape[2]} D{q.shape[3]} b{block} "
          f"items {work.n_items} merges {work.n_merges} slots {work.n_slots}", flush=True)
    o_ref, l_ref = bsa.forward(q, k, v, rp, ci, block, work=work)
    o = torch.full_like(q, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    assert call_noalloc(bsa, q, k, v, rp, ci, block, work, o, lse) == 0
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


def test_noalloc_matches_forward_twice_then_smaller():
    bsa = need_gpu()
    big = case_t2i(bsa)
    check(bsa, big)
    check(bsa, big)
    check(bsa, case_small(bsa))
    check(bsa, big)


def test_noalloc_rejects_oversized_workspace():
    """A work list whose workspace would exceed the static array is refused before any
    launch (host-side check)."""
    bsa = need_gpu()
    q, k, v, rp, ci, block, work = case_small(bsa)
    D = q.shape[3]
    slot = block * (D + 2) * 4
    too_many = bsa.FORWARD_NOALLOC_MAX_BYTES // slot + 1
    assert bsa.forward_workspace_bytes(too_many, D, block) > bsa.FORWARD_NOALLOC_MAX_BYTES
    big = bsa.Work(work.work, work.n_items, work.n_merges, too_many, None, work.max_tiles)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    assert call_noalloc(bsa, q, k, v, rp, ci, block, big, o, lse) == BSA_ERR_CAPACITY
