"""Block-sparse FlashAttention forward and mean-pool top-k mask builder for MI355X.

A thin ctypes binding over libbsa.so (C ABI declared in include/bsa.h).  Every
step of the computation runs in the library's HIP kernels; this module only
checks tensor arguments, allocates outputs and workspaces with torch, and
passes raw pointers plus torch's current HIP stream.  There is no fallback:
if libbsa.so is missing or a call fails, an exception is raised.

Typical use::

    import block_sparse_attention_flashattn_amd as bsa
    row_ptr, col_idx = bsa.build_mask(q, k, block=64, density=0.1)
    o, lse = bsa.forward(q, k, v, row_ptr, col_idx, block=64)

For a fixed shape and static prior, `Plan` precomputes the data-independent
parts once (row_ptr, launch order, device copies of prior and budgets,
workspace) so a step only launches kernels.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

__all__ = [
    "BsaError", "lib", "LIB_PATH", "status_string", "abi_version", "budget_from_density",
    "mask_plan", "work_plan", "validate_csr_host", "build_mask_workspace_bytes",
    "forward_workspace_bytes", "build_mask", "build_mask_status", "schedule", "forward",
    "block_mass", "select_by_mass", "csr_mass", "block_oracle", "residual", "compensate",
    "AnchorReuse", "query_groups", "token_mass", "select_tokens", "gather_forward",
    "backward", "backward_workspace_bytes", "forward_noalloc", "FORWARD_NOALLOC_MAX_BYTES",
    "Plan", "Work", "n_blocks", "default_max_tiles",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

_i32, _i64, _f32, _f64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p
_sz = ctypes.c_size_t

_SIGS = {
    "bsa_status_string": (ctypes.c_char_p, [_i32]),
    "bsa_abi_version": (_i32, []),
    "bsa_budget_from_density": (_i32, [_i32, _f64]),
    "bsa_mask_plan": (_i32, [_i32, _i32, _i32, _f64, _vp, _i32, _vp, _i32, _vp, _vp]),
    "bsa_work_plan_ints": (_i64, [_i32, _i64, _i32]),
    "bsa_work_plan_host": (_i32, [_vp, _i32, _i32, _i32, _i32, _vp, _i64, _vp, _vp, _vp]),
    "bsa_validate_csr_host": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp]),
    "bsa_build_mask_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "bsa_build_mask": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _f64, _vp, _vp, _i32,
                              _i32, _vp, _vp, _vp, _sz, _vp]),
    "bsa_build_mask_status": (_i32, [_vp, _vp, _vp]),
    "bsa_schedule": (_i32, [_vp, _i32, _i32, _vp, _vp]),
    "bsa_forward_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "bsa_forward": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32,
                           _i32, _i32, _f32, _vp, _vp, _vp, _sz, _vp]),
    "bsa_forward_compensated": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                        _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "bsa_forward_noalloc": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                   _i32, _i32, _i32, _f32, _vp, _vp, _vp]),
    "bsa_block_mass": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp]),
    "bsa_select_by_mass": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp, _vp]),
    "bsa_csr_mass": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp, _vp]),
    "bsa_residual": (_i32, [_vp, _vp, _vp, _i64, _vp]),
    "bsa_compensate": (_i32, [_vp, _vp, _vp, _i64, _vp]),
    "bsa_query_groups_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "bsa_query_groups": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "bsa_token_mass": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp]),
    "bsa_select_tokens": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp]),
    "bsa_gather_forward": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _i32,
                                  _f32, _vp, _vp, _vp]),
    "bsa_backward_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i64]),
    "bsa_backward": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                            _i64, _f32, _vp, _vp, _vp, _vp, _sz, _vp]),
}


# BSA_ABI_VERSION of include/bsa.h that these signatures and work-list layouts follow.
ABI_VERSION = 12


class BsaError(RuntimeError):
    """A libbsa entry point returned a non-zero status."""


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m block_sparse_attention_flashattn_amd.build`")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    if handle.bsa_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {handle.bsa_abi_version()}, this binding "
                          f"expects {ABI_VERSION}; rebuild the library")
    return handle


class _Lib:
    """The ctypes handle of libbsa.so, opened at the first call (so that the
    build module can run while the library is missing or stale); a missing or
    mismatched library raises ImportError there."""

    _handle = None

    def __getattr__(self, name):
        if _Lib._handle is None:
            _Lib._handle = _load()
        return getattr(_Lib._handle, name)


lib = _Lib()


def status_string(code: int) -> str:
    return lib.bsa_status_string(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise BsaError(f"{what} failed: {status_string(code)} ({code})")


def abi_version() -> int:
    return lib.bsa_abi_version()


def n_blocks(N: int, block: int) -> int:
    return (N + block - 1) // block


def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _t_ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def budget_from_density(nb: int, density: float) -> int:
    k = lib.bsa_budget_from_density(nb, density)
    if k < 0:
        raise BsaError("bsa_budget_from_density: invalid arguments")
    return k


def _prior_host(prior, B: int, H: int, nb: int):
    if prior is None:
        return None, 0
    p = prior.detach().cpu().numpy() if isinstance(prior, torch.Tensor) else np.asarray(prior)
    p = np.ascontiguousarray(p != 0, dtype=np.uint8)
    if p.shape == (nb, nb):
        return p, 0
    if p.shape == (B, H, nb, nb):
        return p, 1
    raise ValueError(f"prior must be [nb,nb] or [B,H,nb,nb] with nb={nb}, got {p.shape}")


def _budgets_host(budgets, nb: int):
    if budgets is None:
        return None
    b = budgets.detach().cpu().numpy() if isinstance(budgets, torch.Tensor) else np.asarray(budgets)
    b = np.ascontiguousarray(b, dtype=np.int32)
    if b.shape != (nb,):
        raise ValueError(f"budgets must have shape [{nb}], got {b.shape}")
    return b


def mask_plan(B: int, H: int, nb: int, density: float = 0.0, prior=None, budgets=None,
              force_diag: bool = True):
    """Host CSR plan: (row_ptr int32 [B*H*nb+1], nnz)."""
    p, per_head = _prior_host(prior, B, H, nb)
    b = _budgets_host(budgets, nb)
    row_ptr = np.empty(B * H * nb + 1, dtype=np.int32)
    nnz = ctypes.c_int64(0)
    _check(lib.bsa_mask_plan(B, H, nb, float(density), _np_ptr(p), per_head, _np_ptr(b),
                             int(bool(force_diag)), _np_ptr(row_ptr), ctypes.byref(nnz)),
           "bsa_mask_plan")
    return row_ptr, int(nnz.value)


def work_plan(row_ptr, max_tiles: int = 0, nb: int = 0, n_groups: int = 1):
    """Host work list: (work int32 array, n_items, n_merges, n_slots).

    Rows longer than `max_tiles` KV blocks are cut into near-equal chunks
    (max_tiles <= 0: never).  Items come in n_groups groups (heads h with
    h % n_groups == g in group g; one group if n_groups <= 1), head by head and
    longest first inside a head, followed by the merge records, the group
    table {n_groups, start_0, ..., start_n_groups} and the slot map (the merge
    record of every partial slot).
    """
    rp = np.ascontiguousarray(np.asarray(row_ptr), dtype=np.int32)
    n_rows = rp.shape[0] - 1
    cap = int(lib.bsa_work_plan_ints(n_rows, int(rp[-1]), int(max_tiles)))
    if cap < 0:
        raise BsaError("bsa_work_plan_ints: invalid arguments")
    work = np.empty(max(cap, 4), dtype=np.int32)
    ni, nm, ns = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib.bsa_work_plan_host(_np_ptr(rp), n_rows, int(nb), int(max_tiles), int(n_groups),
                                  _np_ptr(work), cap, ctypes.byref(ni), ctypes.byref(nm),
                                  ctypes.byref(ns)), "bsa_work_plan_host")
    tab = 4 * ni.value + 3 * nm.value
    used = tab + 2 + int(work[tab]) + ns.value
    return work[:used].copy(), ni.value, nm.value, ns.value


def validate_csr_host(row_ptr, col_idx, nb: int, strict=True) -> int:
    """-1 if the CSR is well formed, else the first offending row.  strict: True (or 1)
    strictly ascending rows, "distinct" (or 2) distinct columns in any order, False (0)
    columns in range only."""
    rp = np.ascontiguousarray(np.asarray(row_ptr), dtype=np.int32)
    ci = np.ascontiguousarray(np.asarray(col_idx), dtype=np.int32)
    mode = 2 if strict == "distinct" or strict == 2 else int(bool(strict))
    bad = ctypes.c_int64(-1)
    lib.bsa_validate_csr_host(_np_ptr(rp), _np_ptr(ci) if ci.size else None, rp.shape[0] - 1,
                              nb, mode, ctypes.byref(bad))
    return int(bad.value)


def build_mask_workspace_bytes(B: int, H: int, N: int, D: int, block: int) -> int:
    return int(lib.bsa_build_mask_workspace_bytes(B, H, N, D, block))


def forward_workspace_bytes(n_slots: int, D: int, block: int) -> int:
    return int(lib.bsa_forward_workspace_bytes(n_slots, D, block))


def _fwd_lds_bytes(block: int, D: int) -> int:
    """LDS bytes of one forward workgroup, as the kernels allocate them."""
    if block == 64 and D == 64:
        return 40960  # per-wave two-stage K/V rings plus the query staging tile
    tile = block * D * 2
    stages = 3 if tile <= 8192 else 2
    return stages * 2 * tile + (block // 32) * 64 * 2 * 4 + 16


def default_max_tiles(nnz: int, block: int, D: int, n_cu: int, lds_per_cu: int = 160 * 1024):
    """Cut rows longer than 1.5x the average work of one resident workgroup slot.

    A row well above the average keeps its workgroup busy after the others are
    done; cutting it into a few chunks of about that size balances it, while
    every extra chunk costs an epilogue, a partial result and a share of a merge
    (on the t2i mask, text rows cut in two ran faster than in three or five)."""
    slots = n_cu * max(1, lds_per_cu // _fwd_lds_bytes(block, D))
    return max(8, -(-3 * nnz // (2 * slots)))


# Accelerator dies (XCDs) of an MI355X; workgroups are dealt to them round robin.
XCDS = 8


@dataclass
class Work:
    """Device work list of the forward plus the workspace its cut rows need."""
    work: torch.Tensor
    n_items: int
    n_merges: int
    n_slots: int
    workspace: Optional[torch.Tensor]
    max_tiles: int

    @classmethod
    def from_host(cls, row_ptr_host, D: int, block: int, max_tiles: int, device, nb: int = 0,
                  n_groups: int = 1):
        w, ni, nm, ns = work_plan(row_ptr_host, max_tiles, nb, n_groups)
        # The item and merge counters at the start of the workspace must start
        # at zero; every forward call leaves them zero again.
        ws = torch.zeros(forward_workspace_bytes(ns, D, block), dtype=torch.uint8, device=device)
        return cls(torch.from_numpy(w).to(device), ni, nm, ns, ws, int(max_tiles))


def _check_qkv(*ts):
    t0 = ts[0]
    for t in ts:
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError("inputs must be CUDA (HIP) tensors")
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("inputs must be contiguous bf16 [B,H,N,D]")
        if t.shape != t0.shape or t.device != t0.device:
            raise ValueError("inputs must share shape and device")
    return tuple(t0.shape)


def _dev_i32(x, device) -> torch.Tensor:
    if isinstance(x, torch.Tensor):
        if x.dtype != torch.int32 or not x.is_contiguous():
            x = x.to(torch.int32).contiguous()
        return x.to(device)
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x), dtype=np.int32)).to(device)


@dataclass
class Plan:
    """Data-independent CSR plan for one shape, prior and density (host + device copies)."""
    B: int
    H: int
    N: int
    D: int
    block: int
    density: float
    force_diag: bool
    row_ptr_host: np.ndarray
    nnz: int
    row_ptr: torch.Tensor
    work: Work
    prior: Optional[torch.Tensor]
    prior_per_head: int
    budgets: Optional[torch.Tensor]
    workspace: torch.Tensor

    @property
    def nb(self) -> int:
        return n_blocks(self.N, self.block)

    @classmethod
    def create(cls, B, H, N, D, block, density=0.0, prior=None, budgets=None, force_diag=True,
               device="cuda", max_tiles: Optional[int] = None, n_groups: int = XCDS):
        """Host plan of the CSR and of the forward's work list (rows cut at max_tiles;
        None picks `default_max_tiles` for the device, 0 never cuts; items grouped
        by head onto `n_groups` dies, 1 for plain longest-first order)."""
        nb = n_blocks(N, block)
        p, per_head = _prior_host(prior, B, H, nb)
        b = _budgets_host(budgets, nb)
        row_ptr_h, nnz = mask_plan(B, H, nb, density, p, b, force_diag)
        if max_tiles is None:
            n_cu = torch.cuda.get_device_properties(torch.device(device)).multi_processor_count
            max_tiles = default_max_tiles(nnz, block, D, n_cu)
        work = Work.from_host(row_ptr_h, D, block, max_tiles, device, nb, n_groups)
        ws = torch.empty(build_mask_workspace_bytes(B, H, N, D, block), dtype=torch.uint8,
                         device=device)
        return cls(B, H, N, D, block, float(density), bool(force_diag), row_ptr_h, nnz,
                   _dev_i32(row_ptr_h, device), work,
                   None if p is None else torch.from_numpy(p).to(device), per_head,
                   None if b is None else torch.from_numpy(b).to(device), ws)


def build_mask(q: torch.Tensor, k: torch.Tensor, block: int, density: float = 0.0, prior=None,
               budgets=None, force_diag: bool = True, plan: Optional[Plan] = None,
               col_idx: Optional[torch.Tensor] = None):
    """Mean-pool top-k block mask on the GPU -> (row_ptr, col_idx) int32 device tensors.

    Each query block keeps `prior` (+ its diagonal if force_diag) and is filled
    up to its budget (`budgets[i]`, else round(density * nb)) with the KV blocks
    of highest mean-pooled score.  Pass a `Plan` to reuse the host plan.
    """
    B, H, N, D = _check_qkv(q, k)
    if plan is None:
        plan = Plan.create(B, H, N, D, block, density, prior, budgets, force_diag, q.device)
    if (plan.B, plan.H, plan.N, plan.D, plan.block) != (B, H, N, D, block):
        raise ValueError("plan does not match the input shape")
    if col_idx is None:
        col_idx = torch.empty(max(plan.nnz, 1), dtype=torch.int32, device=q.device)
    _check(lib.bsa_build_mask(_t_ptr(q), _t_ptr(k), B, H, N, D, block, plan.density,
                              _t_ptr(plan.budgets), _t_ptr(plan.prior), plan.prior_per_head,
                              int(plan.force_diag), _t_ptr(plan.row_ptr), _t_ptr(col_idx),
                              _t_ptr(plan.workspace), plan.workspace.numel(),
                              _stream_ptr(q.device)), "bsa_build_mask")
    return plan.row_ptr, col_idx


def build_mask_status(plan: Plan) -> int:
    """Synchronously read how many rows disagreed with the plan in the last build."""
    v = ctypes.c_int32(0)
    lib.bsa_build_mask_status(_t_ptr(plan.workspace), _stream_ptr(plan.workspace.device),
                              ctypes.byref(v))
    return int(v.value)


def schedule(row_ptr: torch.Tensor, max_len: int) -> Work:
    """Longest-first work list (no row cut) computed on the device from row_ptr."""
    n_rows = row_ptr.numel() - 1
    work = torch.empty(4 * n_rows + 3, dtype=torch.int32, device=row_ptr.device)
    _check(lib.bsa_schedule(_t_ptr(row_ptr), n_rows, max_len, _t_ptr(work),
                            _stream_ptr(row_ptr.device)), "bsa_schedule")
    # Zeroed item counters (one group, no partial slots); D and block do not
    # change the size of a workspace without partial slots.
    ws = torch.zeros(forward_workspace_bytes(0, 1, 1), dtype=torch.uint8, device=row_ptr.device)
    return Work(work, n_rows, 0, 0, ws, 0)


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, row_ptr, col_idx, block: int,
            scale: Optional[float] = None, work=None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, return_lse: bool = True,
            residual: Optional[torch.Tensor] = None):
    """Block-sparse attention forward -> (O bf16 [B,H,N,D], LSE fp32 [B,H,N] or None).

    `work` is a `Work`, a `Plan` (its work list is used) or None (one workgroup
    per row, natural order).  With `residual` (bf16 [B,H,N,D], not overlapping
    `out`), O = attention + residual, summed in fp32 and rounded once
    (bsa_forward_compensated); LSE stays the attention's.
    """
    B, H, N, D = _check_qkv(q, k, v)
    dev = q.device
    nb = n_blocks(N, block)
    row_ptr = _dev_i32(row_ptr, dev)
    col_idx = _dev_i32(col_idx, dev)
    if row_ptr.numel() != B * H * nb + 1:
        raise ValueError(f"row_ptr must have B*H*nb+1 = {B * H * nb + 1} entries")
    if col_idx.numel() == 0:
        col_idx = torch.zeros(1, dtype=torch.int32, device=dev)
    if isinstance(work, Plan):
        work = work.work
    if work is not None and not isinstance(work, Work):
        raise TypeError("work must be a Work, a Plan or None")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    s = -1.0 if scale is None else float(scale)
    if scale is not None and not s > 0.0:
        raise ValueError("scale must be positive (or None for 1/sqrt(D))")
    if work is None:
        wp, ni, nm, ns, ws, wsb = None, 0, 0, 0, None, 0
    else:
        wp, ni, nm, ns = _t_ptr(work.work), work.n_items, work.n_merges, work.n_slots
        ws = work.workspace
        wsb = 0 if ws is None else ws.numel()
    if residual is None:
        _check(lib.bsa_forward(_t_ptr(q), _t_ptr(k), _t_ptr(v), B, H, N, D, block,
                               _t_ptr(row_ptr), _t_ptr(col_idx), wp, ni, nm, ns, s, _t_ptr(out),
                               _t_ptr(lse) if return_lse else None, _t_ptr(ws), wsb,
                               _stream_ptr(dev)), "bsa_forward")
    else:
        if not isinstance(residual, torch.Tensor) or residual.dtype != torch.bfloat16 \
                or not residual.is_contiguous() or residual.shape != q.shape \
                or residual.device != dev:
            raise ValueError("residual must be a contiguous bf16 [B,H,N,D] tensor on the device")
        _check(lib.bsa_forward_compensated(_t_ptr(q), _t_ptr(k), _t_ptr(v), B, H, N, D, block,
                                           _t_ptr(row_ptr), _t_ptr(col_idx), wp, ni, nm, ns, s,
                                           _t_ptr(residual), _t_ptr(out),
                                           _t_ptr(lse) if return_lse else None, _t_ptr(ws), wsb,
                                           _stream_ptr(dev)), "bsa_forward_compensated")
    return out, (lse if return_lse else None)


# Workspace bytes bsa_forward_noalloc serves (BSA_FORWARD_NOALLOC_MAX_BYTES in bsa.h).
FORWARD_NOALLOC_MAX_BYTES = 16 << 20


def forward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, row_ptr: torch.Tensor,
                    col_idx: torch.Tensor, block: int, out: torch.Tensor, lse: Optional[torch.Tensor],
                    scale: Optional[float] = None, work: Optional["Work"] = None):
    """bsa_forward_noalloc: the forward without a caller workspace (the library's static
    device array serves a work list's counters and partials).  Every argument must already
    be on the device: this wrapper converts and allocates nothing, it only passes pointers."""
    B, H, N, D = _check_qkv(q, k, v)
    for t in (row_ptr, col_idx) + (() if work is None else (work.work,)):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.device != q.device:
            raise ValueError("row_ptr, col_idx and the work list must be int32 device tensors")
    if out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor shaped like q")
    s = -1.0 if scale is None else float(scale)
    wp, ni, nm, ns = (None, 0, 0, 0) if work is None else (
        _t_ptr(work.work), work.n_items, work.n_merges, work.n_slots)
    _check(lib.bsa_forward_noalloc(_t_ptr(q), _t_ptr(k), _t_ptr(v), B, H, N, D, block,
                                   _t_ptr(row_ptr), _t_ptr(col_idx), wp, ni, nm, ns, s,
                                   _t_ptr(out), _t_ptr(lse), _stream_ptr(q.device)),
           "bsa_forward_noalloc")
    return out, lse


def block_mass(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, block: int,
               scale: Optional[float] = None) -> torch.Tensor:
    """Exact attention mass per block pair -> fp32 [B,H,nb,nb].

    mass[b,h,i,j] = sum over queries of block i and keys of block j of
    exp(scale q.k - lse): with the dense LSE (`forward` over an all-ones CSR),
    the block sums of the dense attention probabilities.
    """
    B, H, N, D = _check_qkv(q, k)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be contiguous fp32 [B,H,N]")
    nb = n_blocks(N, block)
    s = -1.0 if scale is None else float(scale)
    if scale is not None and not s > 0.0:
        raise ValueError("scale must be positive (or None for 1/sqrt(D))")
    mass = torch.empty((B, H, nb, nb), dtype=torch.float32, device=q.device)
    _check(lib.bsa_block_mass(_t_ptr(q), _t_ptr(k), _t_ptr(lse), B, H, N, D, block, s,
                              _t_ptr(mass), _stream_ptr(q.device)), "bsa_block_mass")
    return mass


def select_by_mass(mass: torch.Tensor, row_ptr, check: bool = True,
                   nnz: Optional[int] = None) -> torch.Tensor:
    """Block oracle at the density of a CSR: per row, as many blocks as row_ptr gives it,
    the ones of largest mass (ties to the lower block), ascending -> col_idx (device).

    `nnz` (row_ptr's last entry), when the caller knows it, spares a device read;
    `check` waits for the call and raises if a row was longer than nb."""
    if mass.dtype != torch.float32 or not mass.is_contiguous() or mass.dim() < 2:
        raise ValueError("mass must be contiguous fp32 [..., nb]")
    nb = mass.shape[-1]
    n_rows = mass.numel() // nb
    dev = mass.device
    row_ptr = _dev_i32(row_ptr, dev)
    if row_ptr.numel() != n_rows + 1:
        raise ValueError("row_ptr must have one entry per mass row plus one")
    if nnz is None:
        nnz = int(row_ptr[-1].item())
    col_idx = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib.bsa_select_by_mass(_t_ptr(mass), n_rows, nb, _t_ptr(row_ptr), _t_ptr(col_idx),
                                  _t_ptr(status), _stream_ptr(dev)), "bsa_select_by_mass")
    if check and int(status.item()) != 0:
        raise BsaError(f"bsa_select_by_mass: {int(status.item())} rows longer than nb or out of range")
    return col_idx[:nnz]


def csr_mass(mass: torch.Tensor, row_ptr, col_idx) -> torch.Tensor:
    """Retained mass of a CSR per row -> fp32 [n_rows] (device)."""
    if mass.dtype != torch.float32 or not mass.is_contiguous() or mass.dim() < 2:
        raise ValueError("mass must be contiguous fp32 [..., nb]")
    nb = mass.shape[-1]
    n_rows = mass.numel() // nb
    dev = mass.device
    row_ptr = _dev_i32(row_ptr, dev)
    col_idx = _dev_i32(col_idx, dev)
    if row_ptr.numel() != n_rows + 1:
        raise ValueError("row_ptr must have one entry per mass row plus one")
    if col_idx.numel() == 0:
        col_idx = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.empty(n_rows, dtype=torch.float32, device=dev)
    _check(lib.bsa_csr_mass(_t_ptr(mass), n_rows, nb, _t_ptr(row_ptr), _t_ptr(col_idx),
                            _t_ptr(out), _stream_ptr(dev)), "bsa_csr_mass")
    return out


def block_oracle(q: torch.Tensor, k: torch.Tensor, row_ptr, block: int,
                 scale: Optional[float] = None):
    """Two-pass exact block selection at the density of a CSR.

    Pass 1: dense LSE (`forward` over the all-ones CSR).  Pass 2: `block_mass`.
    Then `select_by_mass` with row_ptr's row lengths.  Returns (col_idx, mass).
    """
    B, H, N, D = _check_qkv(q, k)
    nb = n_blocks(N, block)
    dev = q.device
    rows = B * H * nb
    rp1 = torch.arange(rows + 1, dtype=torch.int32, device=dev) * nb
    ci1 = torch.arange(nb, dtype=torch.int32, device=dev).repeat(rows)
    _, lse = forward(q, k, k, rp1, ci1, block, scale=scale)
    mass = block_mass(q, k, lse, block, scale)
    return select_by_mass(mass, row_ptr), mass


def _bf16_pair(a: torch.Tensor, b: torch.Tensor):
    for t in (a, b):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16 \
                or not t.is_contiguous():
            raise ValueError("operands must be contiguous bf16 CUDA (HIP) tensors")
    if a.shape != b.shape or a.device != b.device:
        raise ValueError("operands must share shape and device")


def residual(o_dense: torch.Tensor, o_sparse: torch.Tensor,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """R = O_dense - O_sparse (bf16, formed in fp32, rounded once)."""
    _bf16_pair(o_dense, o_sparse)
    out = torch.empty_like(o_dense) if out is None else out
    _bf16_pair(o_dense, out)
    _check(lib.bsa_residual(_t_ptr(o_dense), _t_ptr(o_sparse), _t_ptr(out), o_dense.numel(),
                            _stream_ptr(o_dense.device)), "bsa_residual")
    return out


def compensate(o_sparse: torch.Tensor, r: torch.Tensor,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """O = O_sparse + R (bf16, formed in fp32, rounded once)."""
    _bf16_pair(o_sparse, r)
    out = torch.empty_like(o_sparse) if out is None else out
    _bf16_pair(o_sparse, out)
    _check(lib.bsa_compensate(_t_ptr(o_sparse), _t_ptr(r), _t_ptr(out), o_sparse.numel(),
                              _stream_ptr(o_sparse.device)), "bsa_compensate")
    return out


class AnchorReuse:
    """Anchor-step reuse with dense-sparse residual compensation.

    `anchor(q, k, v, row_ptr, col_idx, work=None)` runs the dense and the sparse
    forward, keeps the CSR (and work list) and the residual R = O_dense - O_sparse,
    and returns the dense output.  `reuse(q, k, v)` runs the sparse forward with
    the kept CSR and R added in its epilogue (bsa_forward_compensated): O_sparse + R.
    """

    def __init__(self, block: int, scale: Optional[float] = None):
        self.block, self.scale = block, scale
        self.row_ptr = self.col_idx = self.work = self.r = None

    def anchor(self, q, k, v, row_ptr, col_idx, work=None):
        B, H, N, D = _check_qkv(q, k, v)
        nb = n_blocks(N, self.block)
        rows = B * H * nb
        dev = q.device
        rp1 = torch.arange(rows + 1, dtype=torch.int32, device=dev) * nb
        ci1 = torch.arange(nb, dtype=torch.int32, device=dev).repeat(rows)
        o_dense, _ = forward(q, k, v, rp1, ci1, self.block, scale=self.scale, return_lse=False)
        self.row_ptr, self.col_idx, self.work = _dev_i32(row_ptr, dev), _dev_i32(col_idx, dev), work
        o_sparse, _ = forward(q, k, v, self.row_ptr, self.col_idx, self.block, scale=self.scale,
                              work=work, return_lse=False)
        self.r = residual(o_dense, o_sparse, out=o_sparse)
        return o_dense

    def reuse(self, q, k, v, out: Optional[torch.Tensor] = None):
        if self.r is None:
            raise RuntimeError("reuse() before anchor()")
        o, _ = forward(q, k, v, self.row_ptr, self.col_idx, self.block, scale=self.scale,
                       work=self.work, out=out, return_lse=False, residual=self.r)
        return o


def query_groups(q: torch.Tensor, C: int, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Tile-aligned query groups -> int32 [B,H,N/C,C] (token indices, ascending per group)."""
    B, H, N, D = _check_qkv(q)
    if N % C:
        raise ValueError("N must be a multiple of the group size")
    groups = torch.empty((B, H, N // C, C), dtype=torch.int32, device=q.device)
    need = int(lib.bsa_query_groups_workspace_bytes(B, H, N, D, C))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(lib.bsa_query_groups(_t_ptr(q), B, H, N, D, C, _t_ptr(groups), _t_ptr(workspace),
                                workspace.numel(), _stream_ptr(q.device)), "bsa_query_groups")
    return groups


def token_mass(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, groups: torch.Tensor,
               scale: Optional[float] = None) -> torch.Tensor:
    """Per group and KV token, exp(scale q.k - lse) summed over the group's queries
    -> fp32 [B,H,G,N]."""
    B, H, N, D = _check_qkv(q, k)
    if groups.dtype != torch.int32 or not groups.is_contiguous() or groups.dim() != 4 \
            or tuple(groups.shape[:2]) != (B, H):
        raise ValueError("groups must be contiguous int32 [B,H,G,C]")
    G, C = groups.shape[2], groups.shape[3]
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be contiguous fp32 [B,H,N]")
    s = -1.0 if scale is None else float(scale)
    mass = torch.empty((B, H, G, N), dtype=torch.float32, device=q.device)
    _check(lib.bsa_token_mass(_t_ptr(q), _t_ptr(k), _t_ptr(lse), _t_ptr(groups), B, H, N, D, C,
                              s, _t_ptr(mass), _stream_ptr(q.device)), "bsa_token_mass")
    return mass


def select_tokens(mass: torch.Tensor, k: int) -> torch.Tensor:
    """Per mass row, the k tokens of largest mass (ties to the lower token), ascending
    -> int32 [..., k]."""
    if mass.dtype != torch.float32 or not mass.is_contiguous() or mass.dim() < 2:
        raise ValueError("mass must be contiguous fp32 [..., N]")
    N = mass.shape[-1]
    rows = mass.numel() // N
    out = torch.empty(tuple(mass.shape[:-1]) + (k,), dtype=torch.int32, device=mass.device)
    _check(lib.bsa_select_tokens(_t_ptr(mass), rows, N, int(k), _t_ptr(out),
                                 _stream_ptr(mass.device)), "bsa_select_tokens")
    return out


def gather_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, groups: torch.Tensor,
                   tokens: torch.Tensor, scale: Optional[float] = None,
                   out: Optional[torch.Tensor] = None, return_lse: bool = True):
    """Each group's 64 queries attend to exactly that group's tokens -> (O bf16 [B,H,N,D],
    LSE fp32 [B,H,N] or None).  groups int32 [B,H,G,64], tokens int32 [B,H,G,T] (no
    repeats); rows no group names keep the contents of `out` (zeros when it is None)."""
    B, H, N, D = _check_qkv(q, k, v)
    for name, t in (("groups", groups), ("tokens", tokens)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or not t.is_contiguous() \
                or t.dim() != 4 or tuple(t.shape[:2]) != (B, H) or t.device != q.device:
            raise ValueError(f"{name} must be contiguous int32 [B,H,G,...] on q's device")
    G, T = groups.shape[2], tokens.shape[3]
    if groups.shape[3] != 64 or tokens.shape[2] != G:
        raise ValueError("groups must be [B,H,G,64] and tokens [B,H,G,T]")
    if out is None:
        out = torch.zeros_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be contiguous bf16 like q")
    lse = torch.full((B, H, N), float("-inf"), dtype=torch.float32, device=q.device) \
        if return_lse else None
    s = -1.0 if scale is None else float(scale)
    _check(lib.bsa_gather_forward(_t_ptr(q), _t_ptr(k), _t_ptr(v), B, H, N, D, _t_ptr(groups), G,
                                  _t_ptr(tokens), T, s, _t_ptr(out),
                                  _t_ptr(lse) if lse is not None else None,
                                  _stream_ptr(q.device)), "bsa_gather_forward")
    return out, lse


def backward_workspace_bytes(B: int, H: int, N: int, D: int, block: int, nnz: int) -> int:
    return int(lib.bsa_backward_workspace_bytes(B, H, N, D, block, int(nnz)))


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
             lse: torch.Tensor, do: torch.Tensor, row_ptr, col_idx, block: int,
             scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None):
    """dQ, dK, dV (bf16 [B,H,N,D]) of the CSR forward for the incoming gradient `do`, from the
    forward's O and LSE over the same CSR and scale."""
    B, H, N, D = _check_qkv(q, k, v, o, do)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, H, N) \
            or lse.device != q.device:
        raise ValueError("lse must be contiguous fp32 [B,H,N] on q's device")
    rp = _dev_i32(row_ptr, q.device)
    ci = _dev_i32(col_idx, q.device)
    nnz = ci.numel()                 # an upper bound of row_ptr[-1]
    need = backward_workspace_bytes(B, H, N, D, block, nnz)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    s = -1.0 if scale is None else float(scale)
    _check(lib.bsa_backward(_t_ptr(q), _t_ptr(k), _t_ptr(v), _t_ptr(o), _t_ptr(do), _t_ptr(lse),
                            B, H, N, D, block, _t_ptr(rp), _t_ptr(ci) if nnz else None, nnz, s,
                            _t_ptr(dq), _t_ptr(dk), _t_ptr(dv), _t_ptr(workspace),
                            workspace.numel(), _stream_ptr(q.device)), "bsa_backward")
    return dq, dk, dv
