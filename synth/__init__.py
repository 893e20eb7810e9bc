"""Seeded synthetic video-attention inputs.

This module only makes inputs: Q, K, V tensors shaped like the attention of a
video diffusion transformer over a latent grid of frames x height x width, and
(for the variable-budget workload) per-query-block kept-block budgets.  It holds
none of the attention method's arithmetic (no pooling, scores, masking or
attention) and imports nothing from the GPU package or from the oracle, so both
sides can be fed from it.

Recipe (the workloads these pages measure are real Wan2.1 activations, which are
not available; these synthetic tensors stand in for them):

* token order is row-major over the latent grid, n = t*H*W + h*W + w;
* every token vector is iid N(0, 1) noise plus 0.5 x a smooth sinusoidal
  (t, h, w) embedding E: channel c uses axis c mod 3 (t, h or w), j = c // 3,
  frequency f = 1 + ((j // 2) mod 4) cycles over that axis' extent, sin for even
  j and cos for odd j;
* head types:
  - "uniform": Q and K (noise + embedding) are scaled by 0.1;
  - "skewed": the keys of the first 4x4x4 cube of the grid (t<4, h<4, w<4) get
    +strength x u, u a random unit vector drawn per head (strength 4, or drawn
    U(2, 8) per head for the "sink" heads of the extreme-sparsity workload);
  - "local": K = Q + 0.3 x N(0, 1) noise (the K noise draw is reused);
  V is always noise + 0.5 E;
* fp32 values are rounded to bfloat16 (round-to-nearest-even, via torch);
* each (batch, head) has its own numpy Generator seeded with
  [seed, workload id, b, h]; draw order inside a head: Q noise, K noise,
  V noise, then the head's extra draws (unit vector, sink strength);
* variable budgets: c = clamp(floor(exp(U ln(0.2 nblk))), 1, floor(0.2 nblk)),
  U ~ U[0, 1) from a Generator seeded [seed, workload id, 1_000_003].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

CUBE = (4, 4, 4)


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    batch: int
    heads: int
    head_dim: int
    frames: int
    height: int
    width: int
    k_frac: float
    p: float
    head_types: Tuple[str, ...]
    sink_heads: Tuple[int, ...] = ()      # heads whose sink strength ~ U(2, 8)
    variable_budget: bool = False

    @property
    def n_tokens(self) -> int:
        return self.frames * self.height * self.width

    @property
    def grid(self) -> Tuple[int, int, int]:
        return (self.frames, self.height, self.width)

    def n_blocks(self, cube=CUBE) -> int:
        ct, ch, cw = cube
        return (-(-self.frames // ct)) * (-(-self.height // ch)) * (-(-self.width // cw))


def _cycle_types(n: int) -> Tuple[str, ...]:
    order = ("uniform", "skewed", "local")
    return tuple(order[h % 3] for h in range(n))


WORKLOADS = {
    0: Workload(0, "tiny", 1, 2, 64, 4, 16, 16, 0.25, 0.9, ("uniform", "skewed")),
    1: Workload(1, "480p", 1, 12, 128, 21, 30, 52, 0.05, 0.9, _cycle_types(12)),
    2: Workload(2, "720p", 1, 40, 128, 21, 45, 80, 0.03, 0.85, _cycle_types(40)),
    3: Workload(3, "720p-extreme", 1, 40, 128, 21, 45, 80, 0.02, 0.8,
                tuple(["skewed"] * 20) + _cycle_types(40)[20:],
                sink_heads=tuple(range(20))),
    4: Workload(4, "720p-varbudget", 1, 40, 128, 21, 45, 80, 0.0, 0.0,
                _cycle_types(40), variable_budget=True),
}


def custom_workload(batch, heads, head_dim, frames, height, width, k_frac=0.25,
                    p=0.9, head_types: Optional[Sequence[str]] = None,
                    wid: int = 100, name: str = "custom") -> Workload:
    """A workload of arbitrary shape (ragged grids, several batches, d=64/128)."""
    if head_types is None:
        head_types = _cycle_types(heads)
    return Workload(wid, name, batch, heads, head_dim, frames, height, width,
                    k_frac, p, tuple(head_types))


def embedding(frames: int, height: int, width: int, d: int) -> np.ndarray:
    """Smooth sinusoidal (t, h, w) embedding, [N, d] float32, row-major tokens."""
    t, h, w = np.meshgrid(np.arange(frames), np.arange(height), np.arange(width),
                          indexing="ij")
    coords = (t.reshape(-1), h.reshape(-1), w.reshape(-1))
    extent = (frames, height, width)
    out = np.empty((frames * height * width, d), dtype=np.float64)
    for c in range(d):
        axis = c % 3
        j = c // 3
        f = 1 + ((j // 2) % 4)
        arg = 2.0 * math.pi * f * coords[axis] / extent[axis]
        out[:, c] = np.sin(arg) if j % 2 == 0 else np.cos(arg)
    return out.astype(np.float32)


def first_cube_tokens(frames: int, height: int, width: int, cube=CUBE) -> np.ndarray:
    """Row-major token indices of the grid's first cube (t<ct, h<ch, w<cw)."""
    ct, ch, cw = cube
    t, h, w = np.meshgrid(np.arange(min(ct, frames)), np.arange(min(ch, height)),
                          np.arange(min(cw, width)), indexing="ij")
    return (t * height * width + h * width + w).reshape(-1)


def _to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def head_qkv(wl: Workload, b: int, h: int, seed: int = 0,
             emb: Optional[np.ndarray] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """One (batch, head)'s Q, K, V as bfloat16 CPU tensors of shape [N, d]."""
    n, d = wl.n_tokens, wl.head_dim
    if emb is None:
        emb = embedding(wl.frames, wl.height, wl.width, d)
    rng = np.random.default_rng([seed, wl.wid, b, h])
    qn = rng.standard_normal((n, d), dtype=np.float32)
    kn = rng.standard_normal((n, d), dtype=np.float32)
    vn = rng.standard_normal((n, d), dtype=np.float32)
    half_e = np.float32(0.5) * emb
    kind = wl.head_types[h]
    q = qn + half_e
    v = vn + half_e
    if kind == "uniform":
        q = np.float32(0.1) * q
        k = np.float32(0.1) * (kn + half_e)
    elif kind == "skewed":
        k = kn + half_e
        u = rng.standard_normal(d)
        u = (u / np.linalg.norm(u)).astype(np.float32)
        strength = 4.0
        if h in wl.sink_heads:
            strength = float(rng.uniform(2.0, 8.0))
        k[first_cube_tokens(wl.frames, wl.height, wl.width)] += np.float32(strength) * u
    elif kind == "local":
        k = q + np.float32(0.3) * kn
    else:
        raise ValueError(f"unknown head type {kind!r}")
    return _to_bf16(q), _to_bf16(k), _to_bf16(v)


def make_qkv(wl: Workload, seed: int = 0, heads: Optional[Sequence[int]] = None,
             batches: Optional[Sequence[int]] = None):
    """Q, K, V as bfloat16 CPU tensors [B', H', N, d] for the chosen batches/heads."""
    heads = list(range(wl.heads)) if heads is None else list(heads)
    batches = list(range(wl.batch)) if batches is None else list(batches)
    n, d = wl.n_tokens, wl.head_dim
    shape = (len(batches), len(heads), n, d)
    q = torch.empty(shape, dtype=torch.bfloat16)
    k = torch.empty(shape, dtype=torch.bfloat16)
    v = torch.empty(shape, dtype=torch.bfloat16)
    emb = embedding(wl.frames, wl.height, wl.width, d)
    for bi, b in enumerate(batches):
        for hi, h in enumerate(heads):
            q[bi, hi], k[bi, hi], v[bi, hi] = head_qkv(wl, b, h, seed, emb)
    return q, k, v


def row_budgets(wl: Workload, seed: int = 0, cube=CUBE) -> np.ndarray:
    """Per-query-block kept-block counts [B, H, nblk] int32, log-uniform in
    [1, floor(0.2 nblk)], drawn independently of any score."""
    nblk = wl.n_blocks(cube)
    hi = max(1, int(math.floor(0.2 * nblk)))
    rng = np.random.default_rng([seed, wl.wid, 1_000_003])
    u = rng.random((wl.batch, wl.heads, nblk))
    c = np.floor(np.exp(u * math.log(0.2 * nblk)))
    return np.clip(c, 1, hi).astype(np.int32)
