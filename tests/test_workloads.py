"""Counting facts of the synthetic workloads (priors, budgets, planned densities)."""
import numpy as np
import torch

import workloads as W
from oracle import builder as Bd


def test_t2i_prior_counts():
    """128 text + 4096 image tokens at block 64 -> 66 blocks; the image part alone is
    64 blocks per side, i.e. 64 x 64 image block pairs (BSA-DiT §2.1 counts 4096
    tokens at block 64 the same way)."""
    p = W.t2i_prior()
    assert p.shape == (66, 66)
    assert p.sum() == 666                      # 15.29 % of 4356
    assert abs(p.sum() / 66 ** 2 - 0.1529) < 1e-4
    assert p[:2].all() and p[:, :2].all()      # text rows / columns dense
    img = p[2:].sum(1)
    assert img.min() == 7 and img.max() == 9
    assert (np.diag(p) == 1).all()
    assert W.t2i_prior(metric="chebyshev").sum() == 854


def test_video_prior_and_plan():
    p = W.video_prior()
    assert p.shape == (256, 256) and p.sum() == 4840
    assert p.sum(1).min() == 8 and p.sum(1).max() == 27
    counts = Bd.plan_counts(1, 1, 256, 0.10, p, None, True)
    assert counts.sum() == 6728 and Bd.budget(256, 0.10) == 26
    order = W.video_token_order()
    assert np.array_equal(np.sort(order), np.arange(16384))
    t, h, w = order // 1024, (order // 32) % 32, order % 32
    for blk in (0, 77, 255):
        sl = slice(blk * 64, (blk + 1) * 64)
        assert np.ptp(t[sl]) == 3 and np.ptp(h[sl]) == 3 and np.ptp(w[sl]) == 3


def test_ragged_budgets():
    b = W.ragged_budgets()
    assert b.shape == (250,) and b.sum() == 3125 and b.min() == 1 and b.max() == 40
    assert Bd.plan_counts(1, 1, 250, 0.0, None, b, True).sum() == 3125


def test_dynamic_plan():
    assert Bd.plan_counts(1, 1, 128, 0.10, None, None, True).sum() == 1664


def test_tensors_seeded_bf16():
    q1, k1, v1 = W.gaussian_qkv(3, 1, 2, 33, 8)
    q2, _, _ = W.gaussian_qkv(3, 1, 2, 33, 8)
    assert q1.dtype == torch.bfloat16 and torch.equal(q1, q2)
    q, k, v = W.lowrank_qk(2, 1, 1, 256, 16, 64)
    assert q.shape == (1, 1, 256, 16) and q.dtype == torch.bfloat16
    # block-constant structure survives pooling: pooled Q varies across blocks
    pq = q.float().reshape(1, 1, 4, 64, 16).mean(3)
    assert pq.std() > 0.3


def test_config_table():
    assert W.make("t2i").nb == 66 and W.make("video").nb == 256
    assert W.make("ragged").nb == 250 and W.make("ragged_twin").nb == 250
    assert W.make("ragged_twin").N % 128 == 78
