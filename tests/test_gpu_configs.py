"""Full-size workloads in the launch configuration the benchmark times.

The builder is compared row by row with the oracle builder (bit-exact where the
fp64 top-k gap exceeds 1e-4); the forward is compared element by element with the
attention oracle on every CSR row of the benchmark workload (t2i) and on every cut
row plus at least 100 others of the rest, the oracle being fed the GPU's own CSR
so that attention parity does not depend on how ties were broken.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import builder as OB
from parity import compare_attention, compare_csr, need_gpu, sample_rows, token_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["t2i", "dynamic", "video", "ragged", "ragged_twin"])
def test_full_config(name):
    bsa = need_gpu()
    w = W.make(name)
    print(f"config {name}: B{w.B} H{w.H} N{w.N} D{w.D} b{w.block}", flush=True)
    q, k, v = w.tensors()
    prior, budgets = w.prior(), w.budgets()
    plan = bsa.Plan.create(w.B, w.H, w.N, w.D, w.block, w.density, prior, budgets,
                           w.force_diag, "cuda")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    rp, ci = bsa.build_mask(qd, kd, w.block, plan=plan)
    o, lse = bsa.forward(qd, kd, vd, rp, ci, w.block, work=plan)
    torch.cuda.synchronize()
    assert bsa.build_mask_status(plan) == 0
    nb, n_rows = w.nb, w.B * w.H * w.nb
    ci_h = ci.cpu().numpy()[:plan.nnz]
    assert bsa.validate_csr_host(plan.row_ptr_host, ci_h, nb) == -1

    rp_ref, ci_ref, gaps = OB.build_mask(q, k, w.block, w.density, prior, budgets, w.force_diag)
    S = None
    if np.isfinite(gaps).any():
        S = OB.block_scores(OB.mean_pool(q, w.block), OB.mean_pool(k, w.block))
    exact, loose = compare_csr(
        plan.row_ptr_host, ci_h, rp_ref, ci_ref, gaps, nb,
        None if S is None else (lambda r: S[(r // nb) // w.H, (r // nb) % w.H, r % nb]),
        lambda r: OB.prior_row(prior, (r // nb) // w.H, (r // nb) % w.H, r % nb, nb, w.force_diag))
    print(f"csr rows exact {exact} tie-excused {loose}; nnz {plan.nnz} "
          f"density {plan.nnz / (w.B * w.H * nb * nb):.4f}", flush=True)

    # Rows compared with the oracle: every row of the benchmark workload (t2i); for the
    # others every row the work list cuts into chunks plus at least 100 more (the longest,
    # the shortest, each head's partial last block, random ones).
    ni, nm = plan.work.n_items, plan.work.n_merges
    cut = plan.work.work.cpu().numpy()[4 * ni:4 * ni + 3 * nm].reshape(-1, 3)[:, 0]
    if name == "t2i":
        rows = list(range(n_rows))
    else:
        rows = sorted(set(sample_rows(plan.row_ptr_host, nb, n_rows, 100, seed=len(name)))
                      | set(cut.tolist()))
        assert len(rows) >= 100
    O, L = OA.block_sparse_attention(q, k, v, plan.row_ptr_host, ci_h, w.block, w.scale, rows=rows)
    stats = compare_attention(o, lse, O, L, token_rows(rows, nb, w.block, w.N, w.H))
    print(f"attention on {len(rows)} of {n_rows} rows ({len(cut)} cut rows among them): "
          f"{stats}; work items {ni} (max_tiles {plan.work.max_tiles})", flush=True)
