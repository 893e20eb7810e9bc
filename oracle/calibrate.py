"""Top-p calibration of a synthetic workload with the oracle.

    python -m oracle.calibrate --workload 3 --k-frac 0.02 --sparsity 0.97

The seeded synthetic heads are untrained and nearly flat, so Top-p at the
pages' p values keeps far more blocks than trained attention would.  To time
the path at a stated block sparsity with both rules of the hybrid mask active
(SpargeAttention2 summary page, "The Hybrid Top-k+Top-p Masking Rule"), this
script keeps the Top-k fraction and searches for the Top-p threshold, rounded
to three decimals, whose oracle mask over every head of the workload reaches
the target block sparsity (the share of (query block, key block) pairs not
kept).  It prints the threshold and the realised sparsity of the oracle's mask.
Test and benchmark tooling only, like the rest of this package.
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synth  # noqa: E402


def row_cumulative_masses(wl, seed=0):
    """Per head: the row orders' cumulative block probabilities [nblk, nblk]."""
    g = O.Geometry(wl.frames, wl.height, wl.width)
    out = []
    for h in range(wl.heads):
        q, k, _ = synth.head_qkv(wl, 0, h, seed)
        qc, kc = (O.reorder(t.double().numpy(), g) for t in (q, k))
        s = O.block_scores(O.pool(qc, g), O.pool(kc, g), wl.head_dim)
        probs = O.block_softmax(s)
        cums = np.stack([np.cumsum(probs[i][O.rank_order(s[i])]) for i in range(g.nblk)])
        out.append(cums)
    return g, out


def sparsity(cums, kc, p):
    kept = 0
    rows = 0
    n = cums[0].shape[1]
    for c in cums:
        for row in c:
            kept += max(kc, O.top_p_count(row, p))
            rows += 1
    return 1.0 - kept / (rows * n)


def calibrate(wl, k_frac, target, seed=0):
    g, cums = row_cumulative_masses(wl, seed)
    kc = O.ceil_k(k_frac, g.nblk)
    grid = np.round(np.arange(0.0, 1.0005, 0.001), 3)
    # sparsity falls as p rises: the last grid point still at or above target
    # and the first below it bracket it; take the nearer one
    vals = {}
    lo, hi = 0, grid.size - 1
    while hi - lo > 1:
        mid = (lo + hi) // 2
        vals[mid] = sparsity(cums, kc, float(grid[mid]))
        if vals[mid] >= target:
            lo = mid
        else:
            hi = mid
    for i in (lo, hi):
        if i not in vals:
            vals[i] = sparsity(cums, kc, float(grid[i]))
    best = min((lo, hi), key=lambda i: abs(vals[i] - target))
    return float(grid[best]), vals[best], kc


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--k-frac", type=float, default=0.02)
    ap.add_argument("--sparsity", type=float, default=0.97)
    a = ap.parse_args()
    wl = synth.WORKLOADS[a.workload]
    p, sp, kc = calibrate(wl, a.k_frac, a.sparsity)
    print(f"workload {wl.name}: k_frac {a.k_frac} (kc {kc}), p {p:.3f} -> block sparsity {sp:.5f}")


if __name__ == "__main__":
    main()
