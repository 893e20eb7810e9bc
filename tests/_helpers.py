"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same seeded inputs, and compare to the stated bar."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import block_sparse_attention_hybrid_amd as sa
import oracle as O
import synth

# attention output bar for bf16 I/O (oracle's mask fed to the GPU attention)
O_MAX_ABS, O_MEAN_ABS = 2e-2, 2e-3
# LSE bar: float32 online softmax vs float64.  The scores carry at most ~1e-5 of
# float32 rounding (bf16 inputs, 128 products) and the float32 sum of exponentials
# ~1e-7 relative, so 1e-3 / 1e-4 leave about 100x headroom
LSE_MAX_ABS, LSE_MEAN_ABS = 1e-3, 1e-4


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def geom_of(wl: synth.Workload, cube=(4, 4, 4)) -> sa.Geom:
    return sa.make_geom(wl.batch, wl.heads, wl.frames, wl.height, wl.width, wl.head_dim, cube)


def ogeom_of(wl: synth.Workload) -> O.Geometry:
    return O.Geometry(wl.frames, wl.height, wl.width)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def _block_offsets(d: int, v_layout: bool) -> np.ndarray:
    """Element offset inside a 64 x d block of (slot s, dim c), flattened s*d+c,
    for the library's documented QK and V block layouts."""
    s = np.arange(64)[:, None]
    c = np.arange(d)[None, :]
    if v_layout:
        off = ((c // 32) * 4 + s // 16) * 512 + ((s // 8) % 2) * 256 + (c % 32) * 8 + s % 8
    else:
        off = ((s // 32) * (d // 16) + c // 16) * 512 + ((c // 8) % 2) * 256 + (s % 32) * 8 + c % 8
    return off.reshape(-1)


def to_layout(xc: np.ndarray, v_layout: bool) -> np.ndarray:
    """Slot-major cube-major [..., n_pad, d] -> the library's block layout
    (same shape; a pure permutation inside each 64 x d block)."""
    d = xc.shape[-1]
    lead = xc.shape[:-2]
    nblk = xc.shape[-2] // 64
    blocks = xc.reshape(lead + (nblk, 64 * d))
    out = np.empty_like(blocks)
    out[..., _block_offsets(d, v_layout)] = blocks
    return out.reshape(xc.shape)


def row_is_valid(kept: np.ndarray, s_row: np.ndarray, kc: int, p: float) -> bool:
    """A kept list is acceptable at a near tie when it is sorted, unique, in
    range, holds at least kc blocks, reaches the mass p up to the near-tie
    margin, and no dropped block outranks a kept one by more than the margin."""
    n = s_row.size
    if kept.size and (np.any(np.diff(kept) <= 0) or kept[0] < 0 or kept[-1] >= n):
        return False
    if kept.size < min(kc, n):
        return False
    probs = O.block_softmax(s_row)
    if 0 < p < 1 and probs[kept].sum() < p - 2 * O.NEAR_TIE:
        return False
    if p >= 1 and kept.size != n:
        return False
    mask = np.zeros(n, dtype=bool)
    mask[kept] = True
    if mask.all() or not mask.any():
        return True
    margin = O.NEAR_TIE * float(np.max(np.abs(s_row)))
    return s_row[mask].min() >= s_row[~mask].max() - margin


def compare_lists(lut: np.ndarray, counts: np.ndarray, ref: O.MaskResult, p: float):
    """Bit-exact comparison outside near ties; validity inside.  Returns
    (mismatched rows outside near ties, near-tie rows, invalid near-tie rows)."""
    bad, near, invalid = [], 0, []
    B, H, n = counts.shape
    for b in range(B):
        for h in range(H):
            for i in range(n):
                c = int(counts[b, h, i])
                got = lut[b, h, i, :c]
                want = ref.lut[b, h, i, :ref.counts[b, h, i]]
                same = c == ref.counts[b, h, i] and np.array_equal(got, want)
                if ref.near_tie[b, h, i]:
                    near += 1
                    if not row_is_valid(got, ref.scores[b, h, i], int(ref.kc[b, h, i]), p):
                        invalid.append((b, h, i))
                elif not same:
                    bad.append((b, h, i))
    return bad, near, invalid


def attn_errors(o_gpu: np.ndarray, o_ref: np.ndarray, real=None):
    """Max and mean absolute error of O.  For cube-major outputs pass `real`,
    the boolean real-slot mask of the slot axis (second to last): the errors,
    the mean in particular, are then taken over real slots only, since pad
    slots hold exact zeros on both sides and would dilute the mean."""
    if real is not None:
        o_gpu, o_ref = o_gpu[..., real, :], o_ref[..., real, :]
    d = np.abs(o_gpu - o_ref)
    return float(d.max()), float(d.mean())


def grad_errors(got: np.ndarray, want: np.ndarray, real: np.ndarray):
    """Max and mean absolute gradient error over the real slots of cube-major
    gradients [..., n_pad, d], and the largest |gradient| (the relative bar's
    scale)."""
    err = np.abs(got[..., real, :] - want[..., real, :])
    return float(err.max()), float(err.mean()), max(float(np.abs(want).max()), 1e-30)


def lse_errors(l_gpu: np.ndarray, l_ref: np.ndarray):
    fin = np.isfinite(l_ref)
    assert np.array_equal(fin, np.isfinite(l_gpu)), "LSE -inf pattern differs"
    if not fin.any():
        return 0.0, 0.0
    d = np.abs(l_gpu[fin] - l_ref[fin])
    return float(d.max()), float(d.mean())
