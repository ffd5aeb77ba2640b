"""Seeded synthetic inputs shaped like the video / 3D-latent attention workloads.

This module holds no arithmetic of the attention method. It only draws
activations, so both the HIP path and the CPU oracle can be fed the same
tensors. The pages measure on real diffusion models (Wan2.1, MiniMax-H3,
HY3D); none of their weights or data are used. These tensors take only their
shapes (token grid, heads, head dim) and a plausible structure:

* tokens live on a (t, h, w) latent grid, flattened row-major:
  ``n = (t * H + y) * W + x``;
* the grid is cut into spatial blocks ``(bt, bh, bw)`` (edge blocks may be
  partial); blocks are numbered row-major and block ``b`` uses cluster centre
  ``b mod n_centers``;
* per (batch, head) the centres are ``c_k ~ N(0, I_d)``;
* ``Q_i = c(i) + noise * eps``, ``K_i = c(i) + noise * eps'`` (same centre as Q),
  ``V_i = eps''`` with ``eps ~ N(0, 1)``;
* a reuse step t drifts every tensor: ``X_t = X_{t-1} + drift * eps_t``
  (a cumulative random walk applied to the stored values);
* values are drawn in fp32 and stored as bf16 (round to nearest even, by
  torch's conversion); ``dtype=torch.float32`` keeps the fp32 values.

Random streams: one ``numpy.random.Generator`` per (seed, tensor id, batch,
head), seeded through ``SeedSequence``, so any head can be regenerated alone.
Tensor ids: 0 centres, 1/2/3 Q/K/V noise, 16 + 3*t + {0, 1, 2} the Q/K/V drift
of reuse step t (t >= 1).

Layout of every returned tensor: ``[B, N, H, d]``, d contiguous.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_qkv", "drift_qkv", "topk_count", "head_rng"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one attention layer (all heads) and its synthetic structure."""

    name: str
    batch: int
    heads: int
    grid: tuple  # (t, h, w); N = t*h*w
    head_dim: int
    block: tuple  # spatial block of one cluster centre
    group_size: int  # query tile / group size T
    density_pct: int  # nominal density in percent
    noise: float = 0.5
    drift: float = 0.03
    n_centers: int = 8
    reuse_steps: int = 4

    @property
    def seqlen(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def groups(self) -> int:
        return -(-self.seqlen // self.group_size)

    @property
    def topk(self) -> int:
        return topk_count(self.density_pct, self.seqlen)

    def with_density(self, pct: int) -> "Workload":
        return dataclasses.replace(self, density_pct=pct)


def topk_count(density_pct: int, seqlen: int) -> int:
    """Selected keys per group: ceil(pct * N / 100) in integer arithmetic."""
    return (density_pct * seqlen + 99) // 100


# The five workloads: a tiny CPU case, then shapes of Wan2.1-1.3B 480p video,
# Wan2.1-14B 720p video, a long-video single-GPU share and a 3D voxel latent.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, (4, 16, 16), 64, (4, 8, 8), 64, 25, drift=0.05, reuse_steps=1),
    "wan480p": Workload("wan480p", 1, 12, (21, 30, 52), 128, (3, 6, 6), 128, 15, reuse_steps=4),
    "wan720p": Workload("wan720p", 1, 40, (21, 45, 80), 128, (3, 6, 6), 128, 20, drift=0.0, reuse_steps=0),
    "longvideo": Workload("longvideo", 1, 24, (24, 64, 64), 128, (3, 6, 6), 128, 15, reuse_steps=8),
    "voxel3d": Workload("voxel3d", 1, 16, (40, 40, 40), 128, (4, 4, 4), 128, 15, reuse_steps=11),
}


def head_rng(seed: int, tensor_id: int, b: int, h: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tensor_id, b, h]))


def center_ids(grid, block, n_centers) -> np.ndarray:
    """Cluster centre of every token, row-major over the grid."""
    T, H, W = grid
    bt, bh, bw = block
    nby = -(-H // bh)
    nbx = -(-W // bw)
    t = np.arange(T)[:, None, None] // bt
    y = np.arange(H)[None, :, None] // bh
    x = np.arange(W)[None, None, :] // bw
    bid = (t * nby + y) * nbx + x
    return (bid % n_centers).reshape(-1)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _head_qkv(seed, b, h, cid, n_centers, d, noise):
    c = head_rng(seed, 0, b, h).standard_normal((n_centers, d), dtype=np.float32)
    N = cid.shape[0]
    q = c[cid] + np.float32(noise) * head_rng(seed, 1, b, h).standard_normal((N, d), dtype=np.float32)
    k = c[cid] + np.float32(noise) * head_rng(seed, 2, b, h).standard_normal((N, d), dtype=np.float32)
    v = head_rng(seed, 3, b, h).standard_normal((N, d), dtype=np.float32)
    return q, k, v


def _store(arr32: np.ndarray, dtype) -> torch.Tensor:
    t = torch.from_numpy(arr32)
    return t if dtype == torch.float32 else t.to(dtype)


def make_qkv(w: Workload, seed: int = 0, dtype=torch.bfloat16, heads=None):
    """Anchor-step Q, K, V as CPU tensors ``[B, N, H_sel, d]``.

    ``heads`` selects a subset of heads (default all); head h of the subset is
    drawn from the same stream as head h of the full tensor.
    """
    heads = list(range(w.heads)) if heads is None else list(heads)
    N, d = w.seqlen, w.head_dim
    cid = center_ids(w.grid, w.block, w.n_centers)
    out = [torch.empty((w.batch, N, len(heads), d), dtype=dtype) for _ in range(3)]
    jobs = [(b, j, h) for b in range(w.batch) for j, h in enumerate(heads)]

    def run(job):
        b, j, h = job
        for t, a in zip(out, _head_qkv(seed, b, h, cid, w.n_centers, d, w.noise)):
            t[b, :, j, :] = _store(a, dtype)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(run, jobs))
    return tuple(out)


def drift_qkv(w: Workload, prev, step: int, seed: int = 0, heads=None):
    """Reuse-step tensors: ``X_t = store(X_{t-1} + drift * eps_t)`` for X in Q, K, V."""
    heads = list(range(w.heads)) if heads is None else list(heads)
    N, d = w.seqlen, w.head_dim
    dtype = prev[0].dtype
    out = [torch.empty_like(p) for p in prev]
    jobs = [(b, j, h) for b in range(w.batch) for j, h in enumerate(heads)]

    def run(job):
        b, j, h = job
        for x, (src, dst) in enumerate(zip(prev, out)):
            eps = head_rng(seed, 16 + 3 * step + x, b, h).standard_normal((N, d), dtype=np.float32)
            base = src[b, :, j, :].float().numpy()
            dst[b, :, j, :] = _store(base + np.float32(w.drift) * eps, dtype)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(run, jobs))
    return tuple(out)


def small_workload(seqlen: int, heads: int = 1, head_dim: int = 128, group_size: int = 128,
                   density_pct: int = 15, batch: int = 1, name: str = "small") -> Workload:
    """A ragged test shape: the grid is 1 x 1 x N with 1 x 1 x ceil(N/8) blocks,
    so the eight centres each own a contiguous run of tokens."""
    blk = max(1, math.ceil(seqlen / 8))
    return Workload(name, batch, heads, (1, 1, seqlen), head_dim, (1, 1, blk), group_size,
                    density_pct, reuse_steps=1)
