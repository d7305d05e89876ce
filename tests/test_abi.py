"""The C ABI loads, exports every declared symbol, and its host entry points agree
with the oracle's plan.  No GPU needed: device entry points are only called with
arguments they must reject before touching the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_attention_flashattn_amd as bsa
from oracle import builder as Bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "bsa.h")).read()
    return re.findall(r"BSA_API\s+[\w\s\*]+?\b(bsa_\w+)\s*\(", text)


def test_every_declared_symbol_is_exported():
    names = declared_symbols()
    assert len(names) >= 12
    handle = ctypes.CDLL(bsa.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), n
    assert set(names) == set(bsa._SIGS), "binding and header disagree"


def test_status_strings_and_version():
    assert bsa.status_string(0) == "BSA_OK"
    assert bsa.status_string(-1) == "BSA_ERR_INVALID_ARG"
    assert bsa.status_string(-5) == "BSA_ERR_PLAN_MISMATCH"
    assert bsa.status_string(-99) == "BSA_ERR_UNKNOWN"
    assert bsa.abi_version() == bsa.ABI_VERSION == 12


def test_budget_matches_oracle():
    for nb in (1, 7, 8, 64, 66, 128, 250, 256, 1000):
        for d in (0.0, -1.0, 1e-9, 0.01, 0.05, 0.1, 0.15, 0.25, 0.5, 0.999, 1.0, 2.0):
            assert bsa.budget_from_density(nb, d) == Bd.budget(nb, d), (nb, d)
    assert bsa.lib.bsa_budget_from_density(0, 0.5) == -1
    assert bsa.lib.bsa_budget_from_density(8, float("nan")) == -1


@pytest.mark.parametrize("seed", range(4))
def test_mask_plan_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    B, H, nb = 2, 3, int(rng.integers(1, 40))
    density = float(rng.choice([0.0, 0.07, 0.3, 1.0]))
    prior = None
    if seed % 2:
        prior = (rng.random((B, H, nb, nb) if seed == 3 else (nb, nb)) < 0.2).astype(np.uint8)
    budgets = rng.integers(-2, nb + 3, nb) if seed >= 2 else None
    for diag in (True, False):
        rp, nnz = bsa.mask_plan(B, H, nb, density, prior, budgets, diag)
        counts = Bd.plan_counts(B, H, nb, density, prior, budgets, diag)
        assert rp[0] == 0 and np.array_equal(np.diff(rp), counts) and nnz == counts.sum()


def test_mask_plan_workload_totals():
    import workloads as W
    rp, nnz = bsa.mask_plan(2, 24, 66, 0.0, W.t2i_prior())
    assert nnz == 2 * 24 * 666
    rp, nnz = bsa.mask_plan(1, 24, 256, 0.10, W.video_prior())
    assert nnz == 24 * 6728
    rp, nnz = bsa.mask_plan(1, 16, 128, 0.10)
    assert nnz == 16 * 1664
    rp, nnz = bsa.mask_plan(1, 24, 250, 0.0, None, W.ragged_budgets())
    assert nnz == 24 * 3125


def check_work(work, ni, nm, ns, rp, max_tiles, nb=0, n_groups=1):
    """Every row covered exactly once, chunks <= max_tiles, merges consistent, and the
    group table: group g holds the heads h % G == g, chunks of cut rows first, then
    rows; each class head by head, a head's longest items first."""
    lens = np.diff(rp)
    items = work[:4 * ni].reshape(ni, 4).copy()
    items[:, 1] -= rp[items[:, 0]]          # absolute column positions -> positions in the row
    items[:, 2] -= rp[items[:, 0]]
    merges = work[4 * ni:4 * ni + 3 * nm].reshape(nm, 3)
    table = work[4 * ni + 3 * nm:]
    G = int(table[0])
    assert G == (n_groups if nb > 0 and n_groups > 1 else 1) and len(table) == G + 2 + ns
    slot_map = table[G + 2:]
    table = table[:G + 2]
    starts = table[1:]
    assert starts[0] == 0 and starts[-1] == ni and (np.diff(starts) >= 0).all()
    sizes = items[:, 2] - items[:, 1]
    heads = items[:, 0] // nb if nb > 0 else np.zeros(ni, np.int64)
    cut_item = items[:, 3] >= 0
    for g in range(G):
        a, b = starts[g], starts[g + 1]
        c = cut_item[a:b]
        assert (np.diff(c.astype(int)) <= 0).all()          # chunks of cut rows first
        assert (heads[a:b] % G == g).all()
        for cls in (True, False):
            h, sz = heads[a:b][c == cls], sizes[a:b][c == cls]
            assert (np.diff(h) >= 0).all()
            for hv in np.unique(h):
                assert (np.diff(sz[h == hv]) <= 0).all()
    cover = {}
    for row, b, e, slot in items.tolist():
        cover.setdefault(row, []).append((b, e, slot))
    assert sorted(cover) == list(range(len(lens)))
    cut = {m[0]: (m[1], m[2]) for m in merges.tolist()}
    used_slots = []
    for row, parts in cover.items():
        parts.sort()
        assert parts[0][0] == 0 and parts[-1][1] == lens[row]
        assert all(parts[i][1] == parts[i + 1][0] for i in range(len(parts) - 1))
        if row in cut:
            s0, n = cut[row]
            assert len(parts) == n and [p[2] for p in parts] == list(range(s0, s0 + n))
            assert all(e - b <= max_tiles for b, e, _ in parts) and max(e - b for b, e, _ in parts) - min(e - b for b, e, _ in parts) <= 1
            used_slots += list(range(s0, s0 + n))
            m = [i for i, r in enumerate(merges[:, 0].tolist()) if r == row]
            assert len(m) == 1 and (slot_map[s0:s0 + n] == m[0]).all()
        else:
            assert len(parts) == 1 and parts[0][2] == -1
            assert max_tiles <= 0 or lens[row] <= max_tiles
    assert sorted(used_slots) == list(range(ns))


@pytest.mark.parametrize("max_tiles", [0, 1, 3, 8, 100])
def test_work_plan(max_tiles):
    rng = np.random.default_rng(max_tiles)
    lens = rng.integers(0, 30, 300)
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    work, ni, nm, ns = bsa.work_plan(rp, max_tiles)
    check_work(work, ni, nm, ns, rp, max_tiles)
    if max_tiles <= 0:
        assert nm == 0 and ni == 300


@pytest.mark.parametrize("n_groups,n_heads", [(2, 16), (8, 16), (8, 13), (3, 2)])
def test_work_plan_grouped_by_head(n_groups, n_heads):
    """Group g holds the heads h % n_groups == g, walked head by head, longest first."""
    rng = np.random.default_rng(n_groups * 100 + n_heads)
    nb = 10
    lens = rng.integers(0, 25, nb * n_heads)
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    work, ni, nm, ns = bsa.work_plan(rp, 7, nb, n_groups)
    check_work(work, ni, nm, ns, rp, 7, nb, n_groups)


def test_work_plan_groups_may_be_empty():
    rp = np.array([0, 3, 5, 9], np.int32)    # one head of 3 rows, 8 groups
    work, ni, nm, ns = bsa.work_plan(rp, 0, 3, 8)
    assert work[:4 * ni].reshape(ni, 4)[:, 0].tolist() == [2, 0, 1]
    assert work[4 * ni:].tolist() == [8, 0, 3, 3, 3, 3, 3, 3, 3, 3]
    with pytest.raises(bsa.BsaError):
        bsa.work_plan(rp, 0, 3, 65)        # more groups than the forward supports


def test_work_plan_t2i_text_rows_are_cut():
    import workloads as W
    rp, nnz = bsa.mask_plan(2, 24, 66, 0.0, W.t2i_prior())
    work, ni, nm, ns = bsa.work_plan(rp, 16)
    check_work(work, ni, nm, ns, rp, 16)
    assert nm == 96 and ns == 96 * 5 and ni == 3168 - 96 + 480


def test_validate_csr_host():
    rp = np.array([0, 2, 2, 5], np.int32)
    assert bsa.validate_csr_host(rp, np.array([0, 3, 1, 2, 3]), 4) == -1
    assert bsa.validate_csr_host(rp, np.array([0, 4, 1, 2, 3]), 4) == 0      # column out of range
    assert bsa.validate_csr_host(rp, np.array([0, 3, 2, 1, 3]), 4) == 2      # not ascending
    assert bsa.validate_csr_host(rp, np.array([0, 3, 2, 1, 3]), 4, strict=False) == -1
    # distinct columns in any order (a repeated column would count twice in the forward)
    assert bsa.validate_csr_host(rp, np.array([0, 3, 2, 1, 3]), 4, strict="distinct") == -1
    assert bsa.validate_csr_host(rp, np.array([0, 3, 2, 1, 2]), 4, strict="distinct") == 2
    assert bsa.validate_csr_host(rp, np.array([0, 3, 2, 2, 3]), 4, strict="distinct") == 2
    assert bsa.validate_csr_host(rp, np.array([0, 3, 2, 2, 3]), 4, strict=False) == -1
    assert bsa.validate_csr_host(np.array([0, 2, 1], np.int32), np.array([0, 1]), 4) == 1


def test_device_entry_points_reject_bad_arguments():
    L = bsa.lib
    fake = ctypes.c_void_p(4096)      # never dereferenced: every call below fails validation
    odd = ctypes.c_void_p(4097)
    args = lambda q=fake, D=64, blk=64, N=128, ws_bytes=0: (
        q, fake, fake, 1, 1, N, D, blk, fake, fake, fake, 4, 1, 3, 0.125, fake, None, fake,
        ws_bytes, None)
    assert L.bsa_forward(*args(q=None)) == -1
    assert L.bsa_forward(*args(D=96)) == -2
    assert L.bsa_forward(*args(blk=32)) == -2
    assert L.bsa_forward(*args(q=odd)) == -1
    assert L.bsa_forward(*args(N=0)) == -1
    assert L.bsa_forward(*args(ws_bytes=16)) == -4       # counters + 3 partial slots need more
    assert L.bsa_forward(*(args()[:17] + (None, 10 ** 6, None))) == -1   # a work list needs a workspace
    mk = lambda ws_bytes=0, D=64, N=128, ws=fake: L.bsa_build_mask(
        fake, fake, 1, 1, N, D, 64, 0.1, None, None, 0, 1, fake, fake, ws, ws_bytes, None)
    assert mk(ws=None) == -1
    assert mk(D=80) == -2
    assert mk(N=64 * 1025) == -2                      # more than 1024 blocks
    assert mk(ws_bytes=16) == -4                      # workspace too small
    assert L.bsa_schedule(None, 4, 4, fake, None) == -1
    assert L.bsa_schedule(fake, 4, 100000, fake, None) == -2
    assert L.bsa_forward_workspace_bytes(3, 64, 64) == 64 * 4096 + 256 + 3 * 64 * 66 * 4
    assert L.bsa_forward_workspace_bytes(40, 64, 64) == 64 * 4096 + 512 + 40 * 64 * 66 * 4
    assert L.bsa_forward_workspace_bytes(0, 64, 64) == 64 * 4096
    assert L.bsa_build_mask_workspace_bytes(1, 1, 128, 64, 64) >= 256 + 2 * 2 * 64 * 4 + 4 * 4


def test_import_does_not_open_the_library():
    """The package and its build module import without opening libbsa.so (so a
    missing or stale library can be rebuilt); the first call opens it."""
    import subprocess
    import sys
    code = ("import block_sparse_attention_flashattn_amd as b, block_sparse_attention_flashattn_amd.build;"
            "assert b._Lib._handle is None; b.abi_version(); assert b._Lib._handle is not None")
    root = __import__("os").path.dirname(__import__("os").path.dirname(__import__("os").path.abspath(__file__)))
    subprocess.run([sys.executable, "-c", code], check=True, cwd=root)


def test_backward_workspace_bytes():
    L = bsa.lib

    def r256(x):
        return (x + 255) // 256 * 256

    def want(B, H, N, D, nnz):
        # (LSE log2 e, delta) per row, col_ptr [B*H*nb + 1], row_idx [nnz], the column
        # and row splits (int2 [B*H*nb] each), the counter area (576 ints), the two
        # work lists (n_lists = 8 if B*H >= 8 else 1, each ceil(B*H / n_lists) nb
        # max_ch int4 records in each of two parts, max_ch = ceil(nb / chunk)), at
        # D = 128 the transposed position of every entry (nnz ints) and the dS tiles
        # (nnz x 64 x 64 bf16), then the partial slots:
        # chunk = max(16, 2 * ceil(nnz / rows)), 2 nnz / chunk + 1 slots of fp32
        # [dK | dV] (2 x 64 x D x 4 bytes) and as many of dQ (64 x D x 4 bytes);
        # 256-byte rounding.
        nb = -(-N // 64)
        nrow = B * H * nb
        chunk = max(16, 2 * (-(-nnz // nrow)))
        cap = 2 * nnz // chunk + 1
        nl = 8 if B * H >= 8 else 1
        lists = nl * (-(-(B * H) // nl)) * nb * max(1, -(-nb // chunk))
        stored = r256(4 * nnz) + 8192 * nnz if D == 128 else 0
        return (r256(8 * B * H * N) + r256(4 * (nrow + 1)) + r256(4 * nnz) + 2 * r256(8 * nrow)
                + r256(4 * 576) + 2 * r256(32 * lists) + stored
                + cap * 512 * D + cap * 256 * D)

    assert L.bsa_backward_workspace_bytes(1, 2, 512, 64, 64, 100) == want(1, 2, 512, 64, 100) \
        == 651776
    assert L.bsa_backward_workspace_bytes(2, 24, 4224, 64, 64, 31968) == \
        want(2, 24, 4224, 64, 31968)
    assert L.bsa_backward_workspace_bytes(1, 16, 8192, 128, 64, 26624) == \
        want(1, 16, 8192, 128, 26624)
    assert L.bsa_backward_workspace_bytes(0, 2, 512, 64, 64, 100) == 0
    # block 128: the refined 64-block CSR (row pointers, 4 nnz columns) first
    nrow64 = 2 * 24 * (-(-32000 // 64))
    assert L.bsa_backward_workspace_bytes(2, 24, 32000, 128, 128, 5000) == \
        r256(4 * (nrow64 + 1)) + r256(4 * 4 * 5000) + want(2, 24, 32000, 128, 4 * 5000)
