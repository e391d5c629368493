"""Seeded synthetic DiT-shaped attention inputs.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic (no attention, grouping or selection), so both the CPU
oracle (through the tests) and the GPU path (through the tests and the bench)
consume the very same bf16 bytes from here.

Recipe (one attention layer, per head h, in this draw order, fp32):
  centres  c_h ~ N(0, 1)                 [n_clusters, d]
  labels   l   ~ U{0 .. n_clusters-1}    [N]
  Q = c_h[l] + sigma * N(0, 1)           [N, d]
  K = c_h[l] + sigma * N(0, 1)           [N, d]   (same labels as Q)
  V ~ N(0, 1)                            [N, d]
Each reuse step adds drift * N(0, 1) to the fp32 masters of Q, K and V (per
head, Q then K then V) and re-quantises.  fp32 -> bf16 is round-to-nearest-even.
Rows N .. N_pad-1 (padding up to a multiple of the query tile C) are zero.

Label layouts:
  "random" (default)  the uniform draw above: a cluster's tokens are scattered
                      over the whole sequence, so contiguous token blocks mix
                      many clusters (the adversarial case for block layouts).
  "grid"              the same draws are made (so every other value is
                      unchanged), then each token of the latent grid
                      (frames x rows x cols, row-major, the layer's `grid`)
                      takes the label of its spatial cell: the rows x cols
                      plane is cut into cy x cx cells, cy*cx = n_clusters, the
                      same cells in every frame (objects persist over time),
                      so contiguous token blocks see one or two clusters.

The cluster structure stands in for the observation on the MC-Sparse pages that
attention mass concentrates on a small number of token interactions (onedev.kr
summary, section "what it is"); no model weights or dataset items are used.
"""
from __future__ import annotations

import dataclasses
from typing import List

import torch


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    batch: int
    heads: int
    n_valid: int          # tokens N
    head_dim: int         # d
    group_size: int       # query tile C
    density_pct: int      # rho in percent
    n_clusters: int
    sigma: float
    n_reuse: int
    drift: float
    power_iters: int = 20
    seed: int = 0
    grid: tuple = ()          # (frames, rows, cols) of the latent, frames*rows*cols = N
    layout: str = "random"    # "random" or "grid" (see the module docstring)

    @property
    def n_pad(self) -> int:
        c = self.group_size
        return (self.n_valid + c - 1) // c * c

    @property
    def groups(self) -> int:
        return self.n_pad // self.group_size

    @property
    def topk(self) -> int:
        # k = ceil(rho * N), in integer arithmetic
        return (self.n_valid * self.density_pct + 99) // 100

    @property
    def levels(self) -> int:
        g, lv = self.groups, 0
        while (1 << lv) < g:
            lv += 1
        return lv

    @property
    def scale(self) -> float:
        return 1.0 / (self.head_dim ** 0.5)


CONFIGS = {
    "tiny": LayerConfig("tiny", 1, 1, 1024, 64, 64, 25, 16, 0.3, 1, 0.05, grid=(1, 32, 32)),
    "480p": LayerConfig("480p", 1, 24, 32760, 128, 128, 25, 64, 0.3, 4, 0.05, grid=(13, 42, 60)),
    "wan720p": LayerConfig("wan720p", 1, 40, 75600, 128, 128, 15, 64, 0.3, 8, 0.05, grid=(21, 45, 80)),
    "hunyuan720p_15": LayerConfig("hunyuan720p_15", 1, 24, 118800, 128, 128, 15, 128, 0.3, 8, 0.05,
                                  grid=(33, 45, 80)),
    "hunyuan720p_25": LayerConfig("hunyuan720p_25", 1, 24, 118800, 128, 128, 25, 128, 0.3, 8, 0.05,
                                  grid=(33, 45, 80)),
    "3d": LayerConfig("3d", 1, 16, 65536, 64, 128, 15, 256, 0.2, 10, 0.03, grid=(1, 256, 256)),
    # the 480p layer with 96-dimensional heads (another head size of DiT stacks)
    "480p_d96": LayerConfig("480p_d96", 1, 24, 32760, 96, 128, 25, 64, 0.3, 4, 0.05, grid=(13, 42, 60)),
}


def custom(name="custom", batch=1, heads=1, n_valid=512, head_dim=64, group_size=64,
           density_pct=25, n_clusters=8, sigma=0.3, n_reuse=1, drift=0.05, seed=0) -> LayerConfig:
    return LayerConfig(name, batch, heads, n_valid, head_dim, group_size, density_pct,
                       n_clusters, sigma, n_reuse, drift, seed=seed)


def grid_labels(cfg: LayerConfig) -> torch.Tensor:
    """Cluster label of every token under the "grid" layout (int64 [N])."""
    f, rows, cols = cfg.grid
    assert f * rows * cols == cfg.n_valid, "grid does not cover the tokens"
    n = cfg.n_clusters
    cy = max(c for c in range(1, int(n ** 0.5) + 1) if n % c == 0)
    cx = n // cy
    y = torch.arange(rows).repeat_interleave(cols)
    x = torch.arange(cols).repeat(rows)
    cell = (y * cy // rows) * cx + (x * cx // cols)
    return cell.repeat(f)


def _to_bf16_padded(x: torch.Tensor, n_pad: int) -> torch.Tensor:
    b, h, n, d = x.shape
    out = torch.zeros((b, h, n_pad, d), dtype=torch.bfloat16)
    out[:, :, :n] = x.to(torch.bfloat16)
    return out


def generate(cfg: LayerConfig, steps: int | None = None, heads: List[int] | None = None):
    """Return a list of (q, k, v) bf16 CPU tensors [B, H, N_pad, d], one per step.

    Step 0 is the anchor step; steps 1..n are reuse steps with cumulative drift.
    `steps` limits how many steps are produced (default 1 + n_reuse).  `heads`
    restricts the output to a subset of heads; the draws for the other heads are
    still made so that the selected heads' values do not depend on the subset.
    """
    n_steps = 1 + cfg.n_reuse if steps is None else steps
    g = torch.Generator("cpu").manual_seed(cfg.seed)
    B, H, N, d = cfg.batch, cfg.heads, cfg.n_valid, cfg.head_dim
    keep = list(range(H)) if heads is None else list(heads)
    qm = torch.empty((B, len(keep), N, d))
    km = torch.empty_like(qm)
    vm = torch.empty_like(qm)
    for b in range(B):
        for h in range(H):
            centres = torch.randn((cfg.n_clusters, d), generator=g)
            labels = torch.randint(0, cfg.n_clusters, (N,), generator=g)
            if cfg.layout == "grid":
                labels = grid_labels(cfg)
            q = centres[labels] + cfg.sigma * torch.randn((N, d), generator=g)
            k = centres[labels] + cfg.sigma * torch.randn((N, d), generator=g)
            v = torch.randn((N, d), generator=g)
            if h in keep:
                i = keep.index(h)
                qm[b, i], km[b, i], vm[b, i] = q, k, v
    out = [tuple(_to_bf16_padded(t, cfg.n_pad) for t in (qm, km, vm))]
    for _ in range(1, n_steps):
        for b in range(B):
            for h in range(H):
                dq = torch.randn((N, d), generator=g)
                dk = torch.randn((N, d), generator=g)
                dv = torch.randn((N, d), generator=g)
                if h in keep:
                    i = keep.index(h)
                    qm[b, i] += cfg.drift * dq
                    km[b, i] += cfg.drift * dk
                    vm[b, i] += cfg.drift * dv
        out.append(tuple(_to_bf16_padded(t, cfg.n_pad) for t in (qm, km, vm)))
    return out


def sample_groups(cfg: LayerConfig, n_random: int = 6, seed: int = 0) -> List[int]:
    """Groups to check on large configs: first, last and n_random seeded others."""
    G = cfg.groups
    rng = torch.Generator("cpu").manual_seed(seed + 1)
    picks = {0, G - 1}
    while len(picks) < min(G, 2 + n_random):
        picks.add(int(torch.randint(0, G, (1,), generator=rng)))
    return sorted(picks)
