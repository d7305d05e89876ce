#!/usr/bin/env python3
"""Benchmark: block-sparse attention on the text-to-image workload, one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload t2i] [--no-cpu] [--extra]

Workload (default "t2i"): batch 2, 24 heads, N = 4224 (128 text + 4096 image
tokens), head_dim 64, block 64, static modality prior (text dense, image
blocks within manhattan radius 1 on the 8x8 tile grid, 2 anchor blocks):
666 of 4356 block pairs per head (15.29%).

A step is one pass of the hot path over one batch already resident in HBM:
`bsa_build_mask` when the workload has a data-dependent (mean-pool top-k)
part, then `bsa_forward`.  The t2i mask is a static prior, so its CSR and
launch order are planned once, outside the timed steps, as a static mask is
meant to be; the prior-only rebuild is still timed and reported in `extra`.

The JSON line carries:
  value     effective TFLOP/s over active blocks = 4 * q_valid * k_valid * D per
            active block pair, summed, divided by the step time;
  roofline  for bsa_forward (the dominant kernel): algorithmic FLOPs per launch
            / mean launch time (HIP events on the launch stream around one graph
            of back-to-back launches), against the dense bf16 MFMA peak (2.5 PFLOP/s);
  cpu_baseline  the fp64 CPU oracle on a time-bounded sample of whole heads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
HBM_PEAK_GBS = 8000.0
METRIC = "effective TFLOP/s over active blocks + % bf16 MFMA peak, N=4224 t2i mask"
FWD_SRC = os.path.join(ROOT, "block_sparse_attention_flashattn_amd", "csrc", "fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_t2i_traffic.json")


def active_flops(row_ptr, col_idx, N, D, block, nb):
    """Sum over active (query block, key block) pairs of 4 * q_valid * k_valid * D."""
    valid = np.minimum(block, N - np.arange(nb) * block).astype(np.float64)
    rows = np.arange(len(row_ptr) - 1) % nb
    counts = np.diff(row_ptr)
    qv = np.repeat(valid[rows], counts)
    kv = valid[np.asarray(col_idx[: row_ptr[-1]], dtype=np.int64)]
    return float(4.0 * D * np.sum(qv * kv))


def compulsory_bytes(B, H, N, D, nnz, n_rows):
    """Q, K, V read once, O written once (bf16), LSE (fp32), CSR + order (int32)."""
    return float(4 * B * H * N * D * 2 + B * H * N * 4 + (nnz + 2 * n_rows + 1) * 4)


def fwd_kernel_name(block, D):
    """The forward kernel that serves (block, D), as rocprofv3 names it."""
    if block == 64 and D == 64:
        return "bsa_forward (fwd_wide_kernel; cut rows combined inside it)"
    return f"bsa_forward (fwd_kernel<{block}, {D}> + merge_kernel<{block}, {D}>)"


def traffic_for(fwd_sha):
    """HBM bytes per launch from the committed PMC summary, if the kernel is unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("fwd_hip_sha256") != fwd_sha:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, q, k, v, row_ptr, col_idx, budget_s=10.0):
    """Time the fp64 oracle head by head until `budget_s` seconds of CPU work are spent."""
    from oracle import attention as OA
    try:
        from threadpoolctl import threadpool_info
        threads = max([i["num_threads"] for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = os.cpu_count() or 1
    q64, k64, v64 = (x.float().numpy().astype(np.float64) for x in (q, k, v))
    nb = w.nb
    heads, flops, t0 = 0, 0.0, time.perf_counter()
    while heads < w.B * w.H and time.perf_counter() - t0 < budget_s:
        rows = range(heads * nb, (heads + 1) * nb)
        OA.block_sparse_attention(q64, k64, v64, row_ptr, col_idx, w.block, w.scale, rows=rows)
        lo, hi = row_ptr[heads * nb], row_ptr[(heads + 1) * nb]
        sub_rp = row_ptr[heads * nb:(heads + 1) * nb + 1] - lo
        flops += active_flops(sub_rp, col_idx[lo:hi], w.N, w.D, w.block, nb)
        heads += 1
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} heads (all {nb} query blocks each) of the {w.name} "
                      f"workload, fp64 numpy masked softmax, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="t2i")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--extra", action="store_true",
                    help="also time the all-ones (dense) CSR and a density sweep")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run 10 device-to-device copies of this many MiB (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against a copy of known size) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the path shards "
                                   "over (batch, head) with no communication, so multi-GPU "
                                   "figures are not produced", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import block_sparse_attention_flashattn_amd as bsa
    import workloads as W

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.copy_mb > 0:
        n = args.copy_mb * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "copies": 10}))
        return
    dev = "cuda"
    w = W.make(args.workload)
    q, k, v = w.tensors()
    prior, budgets = w.prior(), w.budgets()
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    plan = bsa.Plan.create(w.B, w.H, w.N, w.D, w.block, w.density, prior, budgets, w.force_diag, dev)
    nb, n_rows = w.nb, w.B * w.H * w.nb
    dynamic = w.density > 0 or budgets is not None
    col_idx = torch.empty(max(plan.nnz, 1), dtype=torch.int32, device=dev)
    bsa.build_mask(qd, kd, w.block, plan=plan, col_idx=col_idx)
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    if bsa.build_mask_status(plan) != 0:
        raise RuntimeError("mask plan mismatch")
    ci_h = col_idx.cpu().numpy()[:plan.nnz]
    flops = active_flops(plan.row_ptr_host, ci_h, w.N, w.D, w.block, nb)

    def step():
        if dynamic:
            bsa.build_mask(qd, kd, w.block, plan=plan, col_idx=col_idx)
        bsa.forward(qd, kd, vd, plan.row_ptr, col_idx, w.block, work=plan, out=o, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The K timed steps run as one HIP graph captured beforehand: the host then
    # issues one graph launch instead of K Python calls through the binding (about
    # as long as the forward kernel itself at this size), so the device sets the
    # pace.  One untimed replay uploads the graph.  Eager launches if capture fails.
    graph = None
    try:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                step()
        graph.replay()
        torch.cuda.synchronize()
    except Exception as exc:  # pragma: no cover - depends on the device runtime
        graph = None
        print(f"graph capture failed ({exc}); timing eager launches", file=sys.stderr)
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step_eager = (time.perf_counter() - t0) * 1e3 / args.steps

    # Per-launch forward time with HIP events on the launch stream (torch's current
    # stream): R back-to-back launches in one graph, events around its replay.
    stream = torch.cuda.current_stream()
    reps = max(50, args.steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fwd_graph = None
    if graph is not None:
        fwd_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(fwd_graph):
            for _ in range(reps):
                bsa.forward(qd, kd, vd, plan.row_ptr, col_idx, w.block, work=plan, out=o, lse=lse)
        fwd_graph.replay()
        torch.cuda.synchronize()
    e0.record(stream)
    if fwd_graph is not None:
        fwd_graph.replay()
    else:
        for _ in range(reps):
            bsa.forward(qd, kd, vd, plan.row_ptr, col_idx, w.block, work=plan, out=o, lse=lse)
    e1.record(stream)
    torch.cuda.synchronize()
    fwd_ms = e0.elapsed_time(e1) / reps
    # The same launches one by one, an event pair around each (includes the host's
    # launch latency whenever the device runs ahead of it).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        bsa.forward(qd, kd, vd, plan.row_ptr, col_idx, w.block, work=plan, out=o, lse=lse)
        b.record(stream)
    torch.cuda.synchronize()
    fwd_ms_eager = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    fwd_ms_median = float(np.median([a.elapsed_time(b) for a, b in evs]))

    def time_launches(fn, n=50):
        for _ in range(5):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    build_ms = time_launches(lambda: bsa.build_mask(qd, kd, w.block, plan=plan, col_idx=col_idx))
    achieved = flops / (fwd_ms * 1e-3) / 1e12
    fwd_sha = hashlib.sha256(open(FWD_SRC, "rb").read()).hexdigest()
    extra = {
        "fwd_ms_mean": fwd_ms, "fwd_ms_per_launch_events_mean": fwd_ms_eager,
        "fwd_ms_per_launch_events_median": fwd_ms_median,
        "timed_as_graph": graph is not None, "ms_per_step_eager": ms_per_step_eager,
        "build_mask_ms": build_ms, "build_mask_in_step": dynamic,
        "active_gflop": flops / 1e9, "nnz": plan.nnz,
        "measured_density": plan.nnz / (n_rows * nb),
        "compulsory_mb": compulsory_bytes(w.B, w.H, w.N, w.D, plan.nnz, n_rows) / 1e6,
        "device": torch.cuda.get_device_name(0),
        "cu_count": torch.cuda.get_device_properties(0).multi_processor_count,
    }
    # Exact block selection at this workload's density (two passes: dense LSE, then the
    # block mass; the block oracle keeps the most mass per row), timed per kernel, and
    # the mass and output error of this workload's CSR against it.
    rp_all = torch.arange(n_rows + 1, dtype=torch.int32, device=dev) * nb
    ci_all = torch.arange(nb, dtype=torch.int32, device=dev).repeat(n_rows)
    o_dense = torch.empty_like(qd)
    lse_dense = torch.empty_like(lse)
    dense_once_ms = time_launches(lambda: bsa.forward(qd, kd, vd, rp_all, ci_all, w.block,
                                                      out=o_dense, lse=lse_dense), n=5)
    mass = bsa.block_mass(qd, kd, lse_dense, w.block)
    mass_ms = time_launches(lambda: bsa.block_mass(qd, kd, lse_dense, w.block), n=10)
    ci_or = bsa.select_by_mass(mass, plan.row_ptr)
    select_ms = time_launches(lambda: bsa.select_by_mass(mass, plan.row_ptr, check=False,
                                                                  nnz=plan.nnz), n=10)
    kept_csr = bsa.csr_mass(mass, plan.row_ptr, col_idx[:plan.nnz]).double().sum().item()
    kept_or = bsa.csr_mass(mass, plan.row_ptr, ci_or).double().sum().item()
    o_or = torch.empty_like(qd)
    bsa.forward(qd, kd, vd, plan.row_ptr, ci_or, w.block, out=o_or, lse=None, return_lse=False)
    bsa.forward(qd, kd, vd, plan.row_ptr, col_idx, w.block, work=plan, out=o, lse=lse)
    torch.cuda.synchronize()
    n_q = w.B * w.H * w.N
    def rel_err(a):
        d = (a.float() - o_dense.float()).norm().item()
        return d / max(o_dense.float().norm().item(), 1e-30)
    mass_flops = 2.0 * w.B * w.H * float(w.N) * float(w.N) * w.D   # the QK^T products
    extra["block_oracle"] = {
        "dense_forward_ms": dense_once_ms, "block_mass_ms": mass_ms, "select_ms": select_ms,
        "block_mass_tflops": mass_flops / (mass_ms * 1e-3) / 1e12,
        "block_mass_scores_per_ns": w.B * w.H * float(w.N) ** 2 / (mass_ms * 1e6),
        "mean_kept_mass_csr": kept_csr / n_q, "mean_kept_mass_oracle": kept_or / n_q,
        "rel_err_vs_dense_csr": rel_err(o), "rel_err_vs_dense_oracle": rel_err(o_or),
    }

    # Residual compensation at reuse steps: the two elementwise passes (memory-bound: two
    # bf16 reads and one bf16 write per element) and the anchor and reuse steps.
    r_buf = torch.empty_like(qd)
    n_el = o.numel()
    res_ms = time_launches(lambda: bsa.residual(o_dense, o, out=r_buf), n=20)
    o_c = torch.empty_like(qd)
    comp_ms = time_launches(lambda: bsa.compensate(o, r_buf, out=o_c), n=20)
    ar = bsa.AnchorReuse(w.block)
    anchor_ms = time_launches(lambda: ar.anchor(qd, kd, vd, plan.row_ptr, col_idx, work=plan), n=5)
    reuse_ms = time_launches(lambda: ar.reuse(qd, kd, vd, out=o_c), n=20)
    extra["residual_compensation"] = {
        "residual_ms": res_ms, "compensate_ms": comp_ms,
        "compensate_gbps": 3 * 2 * n_el / (comp_ms * 1e-3) / 1e9,
        "compensate_frac_of_hbm_peak": 3 * 2 * n_el / (comp_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "anchor_step_ms": anchor_ms, "reuse_step_ms": reuse_ms,
    }

    # Token-level selection at the same density: tile-aligned query groups of 64, token
    # mass per group from the dense LSE, the top T tokens per group, and the gathered
    # forward; the kept mass and the output error next to the block CSR's.
    if w.D == 64 and w.N % 64 == 0:
        T = int(round(plan.nnz / (n_rows * nb) * w.N))
        groups = bsa.query_groups(qd, 64)
        grp_ms = time_launches(lambda: bsa.query_groups(qd, 64), n=5)
        tmass = bsa.token_mass(qd, kd, lse_dense, groups)
        tmass_ms = time_launches(lambda: bsa.token_mass(qd, kd, lse_dense, groups), n=10)
        toks = bsa.select_tokens(tmass, T)
        sel_tok_ms = time_launches(lambda: bsa.select_tokens(tmass, T), n=10)
        o_g = torch.zeros_like(qd)
        bsa.gather_forward(qd, kd, vd, groups, toks, out=o_g, return_lse=False)
        gather_ms = time_launches(lambda: bsa.gather_forward(qd, kd, vd, groups, toks, out=o_g,
                                                             return_lse=False), n=20)
        kept_tok = torch.gather(tmass, 3, toks.long()).double().sum().item()
        n_groups = groups.shape[0] * groups.shape[1] * groups.shape[2]
        gather_flops = 4.0 * n_groups * 64 * T * w.D
        extra["token_selection"] = {
            "tokens_per_group": T, "groups": n_groups,
            "query_groups_ms": grp_ms, "token_mass_ms": tmass_ms, "select_tokens_ms": sel_tok_ms,
            "gather_forward_ms": gather_ms,
            "gather_forward_tflops": gather_flops / (gather_ms * 1e-3) / 1e12,
            "mean_kept_mass_tokens": kept_tok / n_q, "mean_kept_mass_csr": kept_csr / n_q,
            "rel_err_vs_dense_tokens": rel_err(o_g), "rel_err_vs_dense_csr": rel_err(o),
        }

    # Backward over the same CSR (block 64, D 64): dQ, dK, dV from the forward's O and LSE
    # for a seeded N(0,1) incoming gradient; 10 * q_valid * k_valid * D FLOPs per active
    # pair (the five products S, dP, dV, dS K, dS^T Q), all four launches in the timing.
    if w.D == 64 and w.block == 64:
        g = torch.Generator("cpu").manual_seed(1000 + w.N)
        do = torch.randn(qd.shape, generator=g, dtype=torch.float32).to(torch.bfloat16).to(dev)
        bws = torch.empty(max(bsa.backward_workspace_bytes(w.B, w.H, w.N, w.block, plan.nnz),
                              256), dtype=torch.uint8, device=dev)
        bsa.backward(qd, kd, vd, o, lse, do, plan.row_ptr, col_idx[:plan.nnz], w.block,
                     workspace=bws)
        bwd_ms = time_launches(lambda: bsa.backward(qd, kd, vd, o, lse, do, plan.row_ptr,
                                                    col_idx[:plan.nnz], w.block,
                                                    workspace=bws), n=20)
        bwd_flops = 2.5 * flops
        extra["backward"] = {
            "backward_ms": bwd_ms, "active_gflop": bwd_flops / 1e9,
            "tflops": bwd_flops / (bwd_ms * 1e-3) / 1e12,
            "frac_of_bf16_peak": bwd_flops / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        }

    if args.extra:
        rp1 =(np.arange(n_rows + 1) * nb).astype(np.int32)
        ci1 = torch.from_numpy(np.tile(np.arange(nb, dtype=np.int32), n_rows)).to(dev)
        rp1d = torch.from_numpy(rp1).to(dev)
        dense_ms = time_launches(lambda: bsa.forward(qd, kd, vd, rp1d, ci1, w.block, out=o, lse=lse))
        dense_flops = active_flops(rp1, ci1.cpu().numpy(), w.N, w.D, w.block, nb)
        extra["dense_ms"] = dense_ms
        extra["dense_tflops"] = dense_flops / (dense_ms * 1e-3) / 1e12
        extra["speedup_vs_dense"] = dense_ms / fwd_ms
        sweep = []
        for d in (0.05, 0.10, 0.15, 0.25, 0.50, 1.0):
            p2 = bsa.Plan.create(w.B, w.H, w.N, w.D, w.block, d, None, None, True, dev)
            rp2, ci2 = bsa.build_mask(qd, kd, w.block, plan=p2)
            t = time_launches(lambda: bsa.forward(qd, kd, vd, rp2, ci2, w.block, work=p2,
                                                  out=o, lse=lse))
            sweep.append({"density": p2.nnz / (n_rows * nb), "nnz": p2.nnz, "fwd_ms": t})
        x = np.array([s["nnz"] for s in sweep], float)
        y = np.array([s["fwd_ms"] for s in sweep])
        slope, icpt = np.polyfit(x, y, 1)
        r2 = 1 - np.sum((y - (slope * x + icpt)) ** 2) / np.sum((y - y.mean()) ** 2)
        extra["density_sweep"] = sweep
        extra["linear_fit"] = {"ms_per_1k_blocks": slope * 1e3, "intercept_ms": icpt, "r2": r2}

    out = {
        "metric": METRIC,
        "value": flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "seq_len": w.N,
                   "head_dim": w.D, "block": w.block, "mask": w.note,
                   "density": plan.nnz / (n_rows * nb)},
        "pct_of_bf16_peak": 100.0 * flops / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic_for(fwd_sha), "kernel": fwd_kernel_name(w.block, w.D),
                     "flops_per_launch": flops},
        "cpu_baseline": None,
        "extra": extra,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, plan.row_ptr_host, ci_h, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
