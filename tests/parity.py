"""Shared helpers for the GPU parity tests (oracle vs libbsa on identical inputs)."""
import math

import numpy as np
import pytest
import torch

# Tolerances fixed for this path: bf16 inputs, fp32 accumulation, bf16 output.
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_ABS = 1e-3
GAP_EXACT = 1e-4


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import block_sparse_attention_flashattn_amd as bsa  # raises if libbsa.so is missing
    return bsa


def token_rows(rows, nb, block, N, H):
    """(b, h, token) index arrays of every valid query token of the given CSR rows."""
    bs, hs, ts = [], [], []
    for r in rows:
        bh, i = divmod(int(r), nb)
        b, h = divmod(bh, H)
        t = np.arange(i * block, min(N, (i + 1) * block))
        bs.append(np.full(t.size, b)); hs.append(np.full(t.size, h)); ts.append(t)
    return np.concatenate(bs), np.concatenate(hs), np.concatenate(ts)


def compare_attention(o_gpu, lse_gpu, O_ref, L_ref, sel):
    """Element-wise comparison on the selected (b, h, token) rows; returns stats."""
    b, h, t = sel
    og = o_gpu.float().cpu().numpy()[b, h, t].astype(np.float64)
    orf = O_ref[b, h, t]
    assert np.isfinite(og).all(), "non-finite output"
    err = np.abs(og - orf)
    stats = {"o_max": float(err.max()), "o_mean": float(err.mean())}
    assert stats["o_max"] <= O_MAX_ABS, stats
    assert stats["o_mean"] <= O_MEAN_ABS, stats
    if lse_gpu is not None:
        lg = lse_gpu.cpu().numpy()[b, h, t].astype(np.float64)
        lr = L_ref[b, h, t]
        inf = np.isneginf(lr)
        assert np.array_equal(np.isneginf(lg), inf)
        if (~inf).any():
            stats["lse_max"] = float(np.abs(lg[~inf] - lr[~inf]).max())
            assert stats["lse_max"] <= LSE_ABS, stats
    return stats


def compare_csr(rp_gpu, ci_gpu, rp_ref, ci_ref, gaps, nb, scores=None, prior_rows=None):
    """Rows with gap > 1e-4 bit-exact; every other row equally long and a valid choice."""
    rp_gpu = np.asarray(rp_gpu, np.int64); rp_ref = np.asarray(rp_ref, np.int64)
    assert np.array_equal(rp_gpu, rp_ref)
    n_rows = rp_ref.size - 1
    exact = loose = 0
    for r in range(n_rows):
        g = np.asarray(ci_gpu[rp_gpu[r]:rp_gpu[r + 1]])
        o = np.asarray(ci_ref[rp_ref[r]:rp_ref[r + 1]])
        assert (np.diff(g) > 0).all() and (g.size == 0 or (g.min() >= 0 and g.max() < nb)), r
        if gaps[r] > GAP_EXACT:
            assert np.array_equal(g, o), (r, g, o, gaps[r])
            exact += 1
        else:
            loose += 1
            assert g.size == o.size
            if scores is not None:
                sel = prior_rows(r)
                fill_g = [j for j in g if not sel[j]]
                out_g = [j for j in range(nb) if j not in set(g.tolist()) and not sel[j]]
                if fill_g and out_g:
                    s = scores(r)
                    assert min(s[fill_g]) >= max(s[out_g]) - GAP_EXACT, r
    return exact, loose


def sample_rows(row_ptr, nb, n_rows, k, seed):
    """A few CSR rows: the longest, the shortest, the last block of a head, and random ones."""
    lens = np.diff(np.asarray(row_ptr))
    rng = np.random.default_rng(seed)
    pick = {int(np.argmax(lens)), int(np.argmin(lens)), nb - 1, n_rows - 1, 0}
    pick |= set(rng.choice(n_rows, size=min(k, n_rows), replace=False).tolist())
    return sorted(pick)
