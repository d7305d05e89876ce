"""Seeded synthetic inputs for block-sparse attention: tensors, static priors, budgets.

This module is shared by the CPU oracle, the tests and the benchmark.  It holds
no part of the method's arithmetic (no pooling, scoring, selection, softmax or
planning): only random tensors and the geometry of the static structural priors
that the method takes as inputs.

Page abbreviations used in citations across this repository:

* BSA-DiT: the article "多模态DiT中的块稀疏注意力：从原理到工程落地"
  (block-sparse attention in multimodal DiTs, from principle to deployment),
  m.nlpx.cn/news/144705.
* MC-Sparse summary: the wispaper.ai research summary "Can sparse attention
  close the quality gap in diffusion transformers", which summarises the paper
  "MC-Sparse: Deconstructing and Closing the Dense-Sparse Attention Gap in
  Diffusion Transformers".

Workloads (sizes fixed by the five benchmark configurations):

* tiny   B1 H2  N512   D64  b64  Bernoulli(0.5) block mask per head, diagonal forced
* t2i    B2 H24 N4224  D64  b64  text + 64x64 image patches, static modality prior
* dynamic B1 H16 N8192 D128 b64  Q/K with block-constant rank-8 structure, top-k 10%
* video  B1 H24 N16384 D128 b64  16x32x32 latent in 4x4x4 cuboids, cuboid prior + top-k to 10%
* ragged B1 H24 N32000 D128 b128 per-row budgets 1..40 (5% overall); twin N31950
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np
import torch

__all__ = [
    "Workload", "CONFIGS", "make", "gaussian_qkv", "lowrank_qk", "tiny_prior",
    "t2i_prior", "video_prior", "ragged_budgets", "n_blocks", "drifting_qkv",
]


def n_blocks(n: int, block: int) -> int:
    """Number of blocks covering n tokens (the last one may be partial)."""
    return (n + block - 1) // block


def gaussian_qkv(seed: int, B: int, H: int, N: int, D: int):
    """Q, K, V drawn fp32 N(0,1) from a seeded CPU generator, then rounded to bf16 (RNE)."""
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (B, H, N, D)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def lowrank_qk(seed: int, B: int, H: int, N: int, D: int, block: int, rank: int = 8):
    """Q, K = iid N(0,1) + block-constant rank-`rank` structure; V = iid N(0,1).

    Q[t] = Z[t] + A_q[t // block] @ W / sqrt(rank), K likewise with A_k and the
    same W, all N(0,1) per head.  The structure is constant inside a block, so it
    survives mean pooling and the block scores vary strongly between pairs.
    """
    g = torch.Generator("cpu").manual_seed(seed)
    nb = n_blocks(N, block)
    shape = (B, H, N, D)
    zq = torch.randn(shape, generator=g, dtype=torch.float32)
    zk = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    aq = torch.randn((B, H, nb, rank), generator=g, dtype=torch.float32)
    ak = torch.randn((B, H, nb, rank), generator=g, dtype=torch.float32)
    w = torch.randn((B, H, rank, D), generator=g, dtype=torch.float32)
    tok_block = torch.arange(N) // block
    sq = (aq @ w) / math.sqrt(rank)  # [B,H,nb,D]
    sk = (ak @ w) / math.sqrt(rank)
    q = zq + sq[:, :, tok_block, :]
    k = zk + sk[:, :, tok_block, :]
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def drifting_qkv(seed: int, steps: int, eps: float, B: int, H: int, N: int, D: int,
                 block: int):
    """Slowly drifting inputs: step t is the block-structured Q, K (lowrank_qk) and V plus
    eps * t times one fixed N(0,1) direction per tensor, rounded to bf16 (RNE).  A list of
    (q, k, v) per step; step 0 is the undrifted base."""
    q0, k0, v0 = (x.float() for x in lowrank_qk(seed, B, H, N, D, block))
    g = torch.Generator("cpu").manual_seed(seed + 1)
    dq, dk, dv = (torch.randn((B, H, N, D), generator=g, dtype=torch.float32) for _ in range(3))
    return [tuple((x + (eps * t) * d).to(torch.bfloat16) for x, d in ((q0, dq), (k0, dk), (v0, dv)))
            for t in range(steps)]


def tiny_prior(seed: int, B: int, H: int, nb: int) -> np.ndarray:
    """Per-head Bernoulli(0.5) block mask, uint8 [B,H,nb,nb] (diagonal forced by the builder)."""
    rng = np.random.default_rng(seed)
    return (rng.random((B, H, nb, nb)) < 0.5).astype(np.uint8)


def t2i_prior(n_text: int = 128, grid: int = 64, block: int = 64, tile: int = 8,
              radius: int = 1, metric: str = "manhattan",
              anchors=((3, 3), (4, 4))) -> np.ndarray:
    """Static text-to-image block prior, uint8 [nb, nb].

    Token order: `n_text` text tokens, then grid x grid image patches stored
    tile-major, so block (n_text/block) + r*S + c holds the tile x tile patch
    square at super-grid cell (r, c), S = grid / tile.

    BSA-DiT §3.1 (modality regions) and §3.2 (local window plus a few global
    tokens): text rows and text columns are dense; image-image pairs are kept
    when the super-grid cells are within `radius` (manhattan or chebyshev); every
    image row also keeps the `anchors` cells as global blocks.
    """
    assert n_text % block == 0 and tile * tile == block
    S = grid // tile
    nt = n_text // block
    nb = nt + S * S
    m = np.zeros((nb, nb), dtype=np.uint8)
    m[:nt, :] = 1
    m[:, :nt] = 1
    cells = [(r, c) for r in range(S) for c in range(S)]
    anchor_ids = [nt + r * S + c for (r, c) in anchors]
    for a, (ra, ca) in enumerate(cells):
        for b, (rb, cb) in enumerate(cells):
            dr, dc = abs(ra - rb), abs(ca - cb)
            d = dr + dc if metric == "manhattan" else max(dr, dc)
            if d <= radius:
                m[nt + a, nt + b] = 1
        for j in anchor_ids:
            m[nt + a, j] = 1
    return m


def video_prior(T: int = 16, Hh: int = 32, Ww: int = 32, ct: int = 4, ch: int = 4,
                cw: int = 4, radius: int = 1) -> np.ndarray:
    """3-D cuboid neighbourhood prior, uint8 [nb, nb] (BSA-DiT §3.2, cuboid attention).

    A T x Hh x Ww latent is cut into ct x ch x cw cuboids; block id =
    (t_c * nH + h_c) * nW + w_c.  Blocks whose cuboid coordinates differ by at
    most `radius` in each of t, h, w are kept.
    """
    nT, nH, nW = T // ct, Hh // ch, Ww // cw
    coords = np.array([(t, h, w) for t in range(nT) for h in range(nH) for w in range(nW)])
    diff = np.abs(coords[:, None, :] - coords[None, :, :]).max(axis=2)
    return (diff <= radius).astype(np.uint8)


def video_token_order(T: int = 16, Hh: int = 32, Ww: int = 32, ct: int = 4, ch: int = 4,
                      cw: int = 4) -> np.ndarray:
    """Raster (t, h, w) index of each token when tokens are ordered cuboid by cuboid.

    Inside a cuboid the order is (t, h, w) lexicographic.  Only used to document
    that every 64-token block is one 4x4x4 cuboid; the iid synthetic tensors do
    not depend on it.
    """
    nH, nW = Hh // ch, Ww // cw
    out = []
    for tc in range(T // ct):
        for hc in range(nH):
            for wc in range(nW):
                for dt in range(ct):
                    for dh in range(ch):
                        for dw in range(cw):
                            t, h, w = tc * ct + dt, hc * ch + dh, wc * cw + dw
                            out.append((t * Hh + h) * Ww + w)
    return np.array(out, dtype=np.int64)


def ragged_budgets(nb: int = 250, lo: int = 1, hi: int = 40, gamma: float = 2.391,
                   seed: int = 4) -> np.ndarray:
    """Uneven per-query-block target counts (BSA-DiT §5.3: per-Q-block target counts).

    k_r = lo + floor((hi - lo) * ((r + 0.5) / nb) ** gamma + 0.5), assigned to
    query blocks by a seeded permutation.  For nb = 250 this sums to 3125
    (5.00% of 250 x 250) with min 1, max 40.
    """
    r = np.arange(nb, dtype=np.float64)
    k = lo + np.floor((hi - lo) * ((r + 0.5) / nb) ** gamma + 0.5)
    perm = np.random.default_rng(seed).permutation(nb)
    out = np.empty(nb, dtype=np.int32)
    out[perm] = k.astype(np.int32)
    return out


@dataclass
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    block: int
    density: float
    force_diag: bool
    seed: int
    kind: str = "gaussian"            # "gaussian" | "lowrank"
    prior_fn: Optional[Callable[[], np.ndarray]] = None
    budgets_fn: Optional[Callable[[], np.ndarray]] = None
    note: str = ""

    @property
    def nb(self) -> int:
        return n_blocks(self.N, self.block)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def tensors(self):
        if self.kind == "lowrank":
            return lowrank_qk(self.seed, self.B, self.H, self.N, self.D, self.block)
        return gaussian_qkv(self.seed, self.B, self.H, self.N, self.D)

    def prior(self) -> Optional[np.ndarray]:
        return None if self.prior_fn is None else self.prior_fn()

    def budgets(self) -> Optional[np.ndarray]:
        return None if self.budgets_fn is None else self.budgets_fn()


CONFIGS = {
    "tiny": Workload("tiny", 1, 2, 512, 64, 64, 0.0, True, 0,
                     prior_fn=lambda: tiny_prior(0, 1, 2, 8),
                     note="per-head Bernoulli(0.5) block mask, diagonal forced"),
    "t2i": Workload("t2i", 2, 24, 4224, 64, 64, 0.0, True, 1,
                    prior_fn=lambda: t2i_prior(),
                    note="128 text + 4096 image tokens; static modality prior only"),
    "dynamic": Workload("dynamic", 1, 16, 8192, 128, 64, 0.10, True, 2, kind="lowrank",
                        note="mean-pool top-k at 10% incl. diagonal"),
    "video": Workload("video", 1, 24, 16384, 128, 64, 0.10, True, 3,
                      prior_fn=lambda: video_prior(),
                      note="cuboid radius-1 prior, filled by mean-pool score to 10%"),
    "ragged": Workload("ragged", 1, 24, 32000, 128, 128, 0.0, True, 4,
                       budgets_fn=lambda: ragged_budgets(),
                       note="per-row budgets 1..40 (5%), mean-pool fill"),
    "ragged_twin": Workload("ragged_twin", 1, 24, 31950, 128, 128, 0.0, True, 4,
                            budgets_fn=lambda: ragged_budgets(),
                            note="N=31950: same 250-block grid, last block 78 valid tokens"),
}


def make(name: str) -> Workload:
    return CONFIGS[name]
