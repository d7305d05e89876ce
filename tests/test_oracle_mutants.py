"""Planted mistakes in the oracle must be caught by its pins.

Each test swaps one oracle step for a plausible wrong version (on the CPU) and
checks that at least one pin test fails.
"""
import numpy as np
import pytest

import test_oracle_attention as TA
import test_oracle_builder as TB
from oracle import attention as A
from oracle import builder as Bd


def fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


ATTN_PINS = [
    (TA.test_all_ones_equals_torch_sdpa, (100, 32)),
    (TA.test_sparse_equals_torch_sdpa_with_token_mask, (77, 16)),
    (TA.test_q_zero_closed_form, ()),
    (TA.test_v_constant, ()),
    (TA.test_hand_two_token, ()),
    (TA.test_hand_gpu_sized, ()),
    (TA.test_rows_sum_to_one_and_lse_bounds, ()),
    (TA.test_empty_row, ()),
]


def any_attn_pin_fails():
    return any(fails(f, *a) for f, a in ATTN_PINS)


def test_unmodified_oracle_passes():
    assert not any_attn_pin_fails()


def test_mutant_skipped_block_as_zero_score(monkeypatch):
    """BSA-DiT §4.3's pitfall: skipped blocks treated as score 0 instead of -inf."""
    monkeypatch.setattr(A, "apply_mask", lambda s, allowed: np.where(allowed, s, 0.0))
    assert any_attn_pin_fails()


def test_mutant_missing_denominator(monkeypatch):
    orig = A.softmax_stats

    def bad(s):
        p, lse = orig(s)
        m = np.where(np.isfinite(s.max(1)), s.max(1), 0.0)
        return np.exp(s - m[:, None]), lse
    monkeypatch.setattr(A, "softmax_stats", bad)
    assert any_attn_pin_fails()


def test_mutant_scale_dropped(monkeypatch):
    monkeypatch.setattr(A, "scores", lambda q, k, scale: q @ k.T)
    assert any_attn_pin_fails()


def test_mutant_transposed_scores(monkeypatch):
    monkeypatch.setattr(A, "scores", lambda q, k, scale: scale * (k @ q.T) if q.shape == k.shape else scale * (q @ k.T))
    assert any_attn_pin_fails()


def test_mutant_lse_base2(monkeypatch):
    orig = A.softmax_stats
    monkeypatch.setattr(A, "softmax_stats", lambda s: (orig(s)[0], orig(s)[1] / np.log(2)))
    assert any_attn_pin_fails()


def test_mutant_off_by_one_block(monkeypatch):
    orig = A.active_blocks
    monkeypatch.setattr(A, "active_blocks", lambda rp, ci, r: np.clip(orig(rp, ci, r) + 1, 0, 10 ** 6))
    assert any_attn_pin_fails()


BUILDER_PINS = [
    (TB.test_hand_block_constant, (8,)),
    (TB.test_hand_block_constant, (7,)),
    (TB.test_partial_block_mean_uses_valid_tokens, ()),
    (TB.test_bruteforce_subsets, (0,)),
    (TB.test_bruteforce_ties_prefer_lower_index, ()),
    (TB.test_density_table, ()),
    (TB.test_invariants, (0,)),
]


def any_builder_pin_fails():
    return any(fails(f, *a) for f, a in BUILDER_PINS)


def test_unmodified_builder_passes():
    assert not any_builder_pin_fails()


def test_mutant_mean_over_full_block(monkeypatch):
    def bad(x, block):
        x = Bd._as64(x)
        B, H, N, D = x.shape
        nb = -(-N // block)
        pad = np.zeros((B, H, nb * block, D)); pad[:, :, :N] = x
        return pad.reshape(B, H, nb, block, D).sum(3) / block
    monkeypatch.setattr(Bd, "mean_pool", bad)
    assert any_builder_pin_fails()


def test_mutant_ties_to_higher_index(monkeypatch):
    orig = Bd.select_row

    def bad(score_row, sel, k_i):
        nb = score_row.shape[0]
        cols, gap = orig(score_row[::-1].copy(), sel[::-1].copy(), k_i)
        return np.sort(nb - 1 - cols), gap
    monkeypatch.setattr(Bd, "select_row", bad)
    assert any_builder_pin_fails()


def test_mutant_ascending_scores(monkeypatch):
    orig = Bd.select_row
    monkeypatch.setattr(Bd, "select_row", lambda s, sel, k: orig(-s, sel, k))
    assert any_builder_pin_fails()


def test_mutant_diagonal_outside_budget(monkeypatch):
    orig = Bd.select_row
    monkeypatch.setattr(Bd, "select_row", lambda s, sel, k: orig(s, sel, k + 1))
    assert any_builder_pin_fails()


def test_mutant_budget_ceil(monkeypatch):
    import math
    monkeypatch.setattr(Bd, "budget", lambda nb, d: 0 if d <= 0 else min(nb, max(1, math.ceil(d * nb))))
    assert any_builder_pin_fails()


def test_mutant_scaled_scores_are_harmless_for_ranking(monkeypatch):
    """A positive scale on the block scores does not change any selection."""
    orig = Bd.block_scores
    monkeypatch.setattr(Bd, "block_scores", lambda pq, pk: 0.125 * orig(pq, pk))
    assert fails(TB.test_hand_block_constant, 8)      # the hand scores are exact integers
    assert not fails(TB.test_bruteforce_subsets, 0)   # but selections are unchanged


# ---- block-mass oracle -------------------------------------------------------
import test_oracle_mass as TM
from oracle import mass as Ms

MASS_PINS = [
    (TM.test_rows_sum_to_query_count, (150, 64)),
    (TM.test_brute_force_tiny, ()),
    (TM.test_equal_keys_give_uniform_mass, ()),
    (TM.test_two_pass_form_matches, ()),
    (TM.test_oracle_csr_hand_row, ()),
    (TM.test_oracle_keeps_the_most_mass, ()),
    (TM.test_full_csr_retains_everything, ()),
]


def any_mass_pin_fails():
    return any(fails(f, *a) for f, a in MASS_PINS)


def test_unmodified_mass_oracle_passes():
    assert not any_mass_pin_fails()


def test_mass_mutant_transposed_probabilities(monkeypatch):
    """Block sums of P^T (queries and keys swapped)."""
    orig = Ms.dense_probabilities
    monkeypatch.setattr(Ms, "dense_probabilities", lambda q, k, s: orig(q, k, s).T.copy())
    assert any_mass_pin_fails()


def test_mass_mutant_normalised_over_queries(monkeypatch):
    """Softmax taken down the columns instead of along each query's row."""
    def bad(q, k, scale):
        s = scale * (Ms._as64(q) @ Ms._as64(k).T)
        e = np.exp(s - s.max(axis=0, keepdims=True))
        return e / e.sum(axis=0, keepdims=True)
    monkeypatch.setattr(Ms, "dense_probabilities", bad)
    assert any_mass_pin_fails()


def test_mass_mutant_scale_dropped(monkeypatch):
    orig = Ms.dense_probabilities
    monkeypatch.setattr(Ms, "dense_probabilities", lambda q, k, s: orig(q, k, 1.0))
    assert any_mass_pin_fails()


def test_mass_mutant_oracle_ties_to_higher_block(monkeypatch):
    def bad(mass, row_ptr):
        m = np.asarray(mass, dtype=np.float64).reshape(-1, mass.shape[-1])
        rp = np.asarray(row_ptr)
        nb = m.shape[1]
        out = []
        for r in range(m.shape[0]):
            order = np.lexsort((-np.arange(nb), -m[r]))
            out.append(np.sort(order[:rp[r + 1] - rp[r]]))
        return np.concatenate(out).astype(np.int32)
    monkeypatch.setattr(Ms, "oracle_csr", bad)
    assert any_mass_pin_fails()


def test_mass_mutant_oracle_smallest_first(monkeypatch):
    def bad(mass, row_ptr):
        m = np.asarray(mass, dtype=np.float64).reshape(-1, mass.shape[-1])
        rp = np.asarray(row_ptr)
        nb = m.shape[1]
        return np.concatenate([np.sort(np.lexsort((np.arange(nb), m[r]))[:rp[r + 1] - rp[r]])
                               for r in range(m.shape[0])]).astype(np.int32)
    monkeypatch.setattr(Ms, "oracle_csr", bad)
    assert any_mass_pin_fails()


# ---- residual-compensation oracle --------------------------------------------
import test_oracle_residual as TR
from oracle import residual as Rs

RES_PINS = [
    (TR.test_anchor_step_is_exact, ()),
    (TR.test_zero_drift_reuses_exactly, ()),
    (TR.test_all_ones_csr_has_zero_residual, ()),
    (TR.test_small_drift_compensation_beats_sparse, ()),
    (TR.test_residual_sign, ()),
]


def any_res_pin_fails():
    return any(fails(f, *a) for f, a in RES_PINS)


def test_unmodified_residual_oracle_passes():
    assert not any_res_pin_fails()


def test_res_mutant_residual_sign_flipped(monkeypatch):
    monkeypatch.setattr(Rs, "residual", lambda d, s: np.asarray(s, float) - np.asarray(d, float))
    assert any_res_pin_fails()


def test_res_mutant_compensation_subtracts(monkeypatch):
    monkeypatch.setattr(Rs, "compensate", lambda s, r: np.asarray(s, float) - np.asarray(r, float))
    assert any_res_pin_fails()


# ---- token-level selection oracle ----------------------------------------------
import test_oracle_tokensel as TT
from oracle import tokensel as Tk

TOK_PINS = [
    (TT.test_principal_direction_is_the_top_eigenvector, ()),
    (TT.test_partition_is_exact_and_tile_sized, ()),
    (TT.test_separated_clusters_are_recovered, ()),
    (TT.test_odd_group_count_cuts_at_a_tile_boundary, ()),
    (TT.test_token_mass_conservation_and_block_sums, ()),
    (TT.test_select_tokens_hand, ()),
    (TT.test_gathered_attention_reduces_to_dense_and_block_sparse, ()),
    (TT.test_power_iteration_hand_golden, ()),
]


def any_tok_pin_fails():
    return any(fails(f, *a) for f, a in TOK_PINS)


def test_unmodified_tokensel_oracle_passes():
    assert not any_tok_pin_fails()


def test_tok_mutant_direction_is_a_fixed_axis(monkeypatch):
    """Projecting on the first coordinate instead of the principal direction."""
    monkeypatch.setattr(Tk, "principal_direction",
                        lambda x, iters=None: np.eye(x.shape[1])[0])
    assert any_tok_pin_fails()


@pytest.mark.parametrize("iters", [7, 9])
def test_tok_mutant_power_iteration_count(monkeypatch, iters):
    monkeypatch.setattr(Tk, "POWER_ITERS", iters)
    assert any_tok_pin_fails()


@pytest.mark.parametrize("start", ["ones", "d_over_D_minus_1", "descending"])
def test_tok_mutant_start_vector(monkeypatch, start):
    f = {"ones": lambda D: np.ones(D),
         "d_over_D_minus_1": lambda D: 1.0 + np.arange(D) / max(D - 1, 1),
         "descending": lambda D: 1.0 + np.arange(D)[::-1] / D}[start]
    monkeypatch.setattr(Tk, "start_vector", f)
    assert any_tok_pin_fails()


def test_tok_mutant_mass_summed_over_keys(monkeypatch):
    monkeypatch.setattr(Tk, "token_mass", lambda q, k, groups, scale: np.stack(
        [Tk.M.dense_probabilities(q, k, scale)[:, g].sum(axis=1) for g in np.asarray(groups)]))
    assert any_tok_pin_fails()


def test_tok_mutant_selects_smallest(monkeypatch):
    monkeypatch.setattr(Tk, "select_tokens", lambda m, k: np.stack(
        [np.sort(np.lexsort((np.arange(m.shape[1]), r))[:k]) for r in np.asarray(m)]))
    assert any_tok_pin_fails()


# ---- backward oracle -----------------------------------------------------------
import test_oracle_backward as TBW
from oracle import backward as Bw

BWD_PINS = [
    (TBW.test_closed_forms, ()),
    (TBW.test_sparse_equals_torch_autograd_with_token_mask, ()),
    (TBW.test_dense_equals_torch_autograd, (64, 16)),
    (TBW.test_finite_differences, ()),
]


def any_bwd_pin_fails():
    return any(fails(f, *a) for f, a in BWD_PINS)


def test_unmodified_backward_oracle_passes():
    assert not any_bwd_pin_fails()


def test_bwd_mutant_delta_dropped(monkeypatch):
    monkeypatch.setattr(Bw, "delta", lambda do, o: np.zeros(do.shape[0]))
    assert any_bwd_pin_fails()


def test_bwd_mutant_delta_averaged(monkeypatch):
    monkeypatch.setattr(Bw, "delta", lambda do, o: (do * o).mean(axis=1))
    assert any_bwd_pin_fails()


def test_bwd_mutant_score_gradient_without_p(monkeypatch):
    monkeypatch.setattr(Bw, "score_gradient", lambda p, dp, dl: dp - dl[:, None])
    assert any_bwd_pin_fails()


def test_bwd_mutant_score_gradient_sign(monkeypatch):
    monkeypatch.setattr(Bw, "score_gradient", lambda p, dp, dl: p * (dl[:, None] - dp))
    assert any_bwd_pin_fails()


def test_bwd_mutant_mask_ignored(monkeypatch):
    orig = Bw.probabilities
    monkeypatch.setattr(Bw, "probabilities",
                        lambda q, k, allowed, scale: orig(q, k, np.ones_like(allowed), scale))
    assert any_bwd_pin_fails()
