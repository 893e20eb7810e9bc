#!/usr/bin/env python3
"""Throughput of the hybrid block-sparse attention hot path on one MI355X.

One step = the whole path on one batch of resident synthetic input:
reorder Q and K (pooling them on the way) and V -> float32 block scores ->
hybrid selection -> block-sparse forward writing O and LSE back in token order
(the inverse re-indexing fused into its epilogue), all HIP kernels of
libsparse_attn.so called through the C ABI.

Headline workload: Wan2.1-14B-720p-shaped attention, B=1, H=40, d=128, latent
grid 21x45x80 (75,600 tokens, 1,440 cubes of 4x4x4), Top-k 3% (the pages'
value) and Top-p 0.073, which realises 95.0% block sparsity on these inputs
with both rules active.  value = kept-block attention FLOPs (4*64*64*d per
kept query-block/key-block pair) / step time.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
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
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_sparse_attention_hybrid_amd as sa  # noqa: E402
import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
PEAK_FP64_TFLOPS = 78.6        # MI355X float64 (vector and matrix)
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X float32 matrix cores

# HBM-side traffic of the forward kernel, measured by rocprofv3 counters and
# recorded with a hash of the sources it was measured on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kernels_720p-hybrid95_hbm_traffic.txt")
FWD_SOURCES = ("block_sparse_attention_hybrid_amd/csrc/fwd.hip", "block_sparse_attention_hybrid_amd/csrc/sa_device.h",
               "block_sparse_attention_hybrid_amd/csrc/sa_launch.h", "block_sparse_attention_hybrid_amd/csrc/sa_rowmap.h",
               "block_sparse_attention_hybrid_amd/build.py")

# name -> (synthetic workload id, k_frac, p, row budgets?).  The p of the
# hybrid95 and 97 workloads is the oracle-calibrated Top-p threshold that
# realises 95.0% / 97.0% block sparsity with the pages' Top-k fraction
# (python -m oracle.calibrate --workload 2 --k-frac 0.03 --sparsity 0.95, and
# --workload 3 --k-frac 0.02 --sparsity 0.97)
WORKLOADS = {
    "720p-hybrid95": (2, 0.03, 0.073, False),
    "720p-97": (3, 0.02, 0.052, False),
    "720p-literal": (2, 0.03, 0.85, False),
    "720p-extreme": (3, 0.02, 0.8, False),
    "720p-varbudget": (4, 0.0, 0.0, True),
    "480p": (1, 0.05, 0.9, False),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="720p-hybrid95", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--serial", action="store_true",
                    help="launch the stages from Python one after another instead of the library's "
                         "whole-path call")
    ap.add_argument("--overlap", type=int, default=-1, metavar="ROWS",
                    help="two streams: re-indexing beside the scores and selection, and the forward in "
                         "chunks of ROWS batch*head rows with each chunk's output re-indexed beside the "
                         "next (-1: one chunk); 0 uses one stream")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip timing the coarse-output and router kernels")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the forward timings on the other workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


class Path:
    """Buffers and calls of one step."""

    def __init__(self, wl, k_frac, p, budgets, dev):
        self.wl, self.k_frac, self.p = wl, k_frac, p
        self.g = sa.make_geom(wl.batch, wl.heads, wl.frames, wl.height, wl.width, wl.head_dim)
        self.nblk, self.n_real, self.n_pad = sa.sparse_attn_geometry(self.g)
        t0 = time.time()
        q, k, v = synth.make_qkv(wl, 0)
        log(f"[bench] inputs generated in {time.time() - t0:.1f}s")
        self.q, self.k, self.v = (t.to(dev) for t in (q, k, v))
        del q, k, v
        B, H, d, n = wl.batch, wl.heads, wl.head_dim, self.nblk
        shape_c = (B, H, self.n_pad, d)
        self.qc, self.kc, self.vc, self.oc = (torch.empty(shape_c, dtype=torch.bfloat16, device=dev)
                                              for _ in range(4))
        self.o = torch.empty((B, H, self.n_real, d), dtype=torch.bfloat16, device=dev)
        self.lse_c = torch.empty((B, H, self.n_pad), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, H, self.n_real), dtype=torch.float32, device=dev)
        gen = torch.Generator(device="cpu").manual_seed(7)
        self.o_grad = torch.randn((B, H, self.n_real, d), generator=gen).to(torch.bfloat16).to(dev)
        self.cap = n
        self.lut = torch.empty((B, H, n, n), dtype=torch.int32, device=dev)
        self.counts = torch.empty((B, H, n), dtype=torch.int32, device=dev)
        self.qbar, self.kbar = (torch.empty((B, H, n, d), dtype=torch.float64, device=dev) for _ in range(2))
        self.scores = torch.empty((B, H, n, n), dtype=torch.float64, device=dev)   # path workspace; float64 rows
        self.scores32 = torch.empty((B, H, n, n), dtype=torch.float32, device=dev)
        self.rb = None
        if budgets:
            self.rb = torch.from_numpy(synth.row_budgets(wl, 0)).to(dev)
        nfw = sa.sparse_attn_fwd_workspace_bytes(self.g)
        self.fws = torch.empty(max(nfw, 256), dtype=torch.uint8, device=dev)
        ptr = lambda t: t.data_ptr()
        self.buf = sa.PathBuffers(ptr(self.q), ptr(self.k), ptr(self.v), ptr(self.qc), ptr(self.kc), ptr(self.vc),
                                  ptr(self.qbar), ptr(self.kbar), ptr(self.scores), ptr(self.lut),
                                  ptr(self.counts), self.cap, None if self.rb is None else ptr(self.rb),
                                  None, None, ptr(self.o), ptr(self.lse))   # token order straight from the forward
        self.aux = torch.cuda.Stream(device=dev)

    def stages(self):
        g = self.g
        return [
            ("reorder", lambda: sa.sparse_attn_reorder_qkv(self.q, self.k, self.v, self.qc, self.kc, self.vc,
                                                           self.qbar, self.kbar, g)),
            # float32 block scores and the selection on them, as the whole-path call runs them
            ("mask", lambda: (sa.sparse_attn_block_scores_f32(self.qbar, self.kbar, self.scores32, 0.0, g),
                              sa.sparse_attn_select_f32(self.scores32, g, self.k_frac, self.p, self.rb, self.lut,
                                                    self.counts, self.cap))),
            # the forward with the inverse re-indexing fused (O and LSE in token order)
            # (the count-balanced row order where per-row budgets are given, as the whole-path call does)
            ("fwd", lambda: sa.sparse_attn_fwd_tokens(self.qc, self.kc, self.vc, self.lut, self.counts, self.cap,
                                                      g, 0.0, self.o, self.lse,
                                                      self.fws if self.rb is not None else None)),
        ]

    def step(self):
        for _, fn in self.stages():
            fn()

    def step_call(self, overlap_rows):
        """The whole path as one library call (sparse_attn_attention).  With
        overlap_rows != 0 it runs on two streams: re-indexing beside the scores
        and selection, then the forward in chunks of overlap_rows rows (all rows
        when negative) with each chunk's output re-indexed beside the next."""
        rows = self.g.batch * self.g.heads
        chunk = rows if overlap_rows < 0 else max(1, overlap_rows)
        sa.sparse_attn_attention(self.buf, self.g, self.k_frac, self.p, 0.0, chunk,
                                 aux_stream=self.aux.cuda_stream if overlap_rows != 0 else None)


def fwd_source_hash():
    h = hashlib.sha256()
    for rel in FWD_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """Bytes per forward launch from the committed counter summary, or None when
    it was taken on another workload or on different kernel sources."""
    if workload != "720p-hybrid95" or not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and parts[0] in ("traffic_bytes_per_launch", "fwd_source_sha256"):
                vals[parts[0]] = parts[1]
    if vals.get("fwd_source_sha256") != fwd_source_hash() or "traffic_bytes_per_launch" not in vals:
        return None
    return int(float(vals["traffic_bytes_per_launch"]))


def min_bytes(path):
    """The least HBM traffic of the mask path (per step), independent of how
    it is built: Q, K and V each read once in token order and written once in
    cube order (the pooling fused into that read), the block scores written
    once and read once at float32 size, and the lists (counts and kept ids)
    written once."""
    wl = path.wl
    B, H, d, n = wl.batch, wl.heads, wl.head_dim, path.nblk
    tok = 2 * d
    kept = int(path.counts.sum().item())
    return {"reorder": B * H * 3 * (path.n_real + path.n_pad) * tok,
            "mask": B * H * (n * n * 4 * 2 + n * 4) + kept * 4}


def algorithmic_bytes(path):
    """HBM bytes each stage of this implementation moves at minimum (per
    step): as min_bytes, plus the float64 block means written by the
    re-indexing and read by the scores (the scores are float32, as in
    min_bytes)."""
    wl = path.wl
    B, H, d, n = wl.batch, wl.heads, wl.head_dim, path.nblk
    real, pad = path.n_real, path.n_pad
    tok = 2 * d                                        # bf16 row bytes
    kept = int(path.counts.sum().item())
    return {
        "reorder": B * H * (3 * (real + pad) * tok            # Q, K, V read and written
                            + 2 * n * d * 8),                 # Qbar, Kbar written
        "mask": (B * H * (2 * n * d * 8                       # Qbar, Kbar read
                          + n * n * 4 * 2                     # float32 scores written and read
                          + n * 4) + kept * 4),               # counts + kept ids
    }


def time_call(fn, reps):
    """Mean event-timed duration (ms) of fn on the current stream."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def next_rows(path, reps=3):
    """Kernels beyond the timed step (coarse branch output, fine-grained
    router), timed on the same resident inputs; not part of `value`."""
    wl, g, n = path.wl, path.g, path.nblk
    B, H, d = wl.batch, wl.heads, wl.head_dim
    dev = path.q.device
    vbar = torch.empty((B, H, n, d), dtype=torch.float64, device=dev)
    ocb = torch.empty_like(vbar)
    out = {}
    # the rows below take the float64 block scores (the path's workspace holds float32 ones)
    sa.sparse_attn_block_scores(path.qbar, path.kbar, path.scores, 0.0, g)
    t_vpool = time_call(lambda: sa.sparse_attn_reorder_pool(path.v, path.vc, sa.SA_LAYOUT_V, vbar, g), reps)
    t_coarse = time_call(lambda: sa.sparse_attn_coarse(path.scores, vbar, ocb, g), reps)
    fl = 2.0 * B * H * n * n * d
    out["coarse"] = {"ms": round(t_coarse, 4), "tflops_fp64": round(fl / t_coarse / 1e9, 2),
                     "frac_of_fp64_peak": round(fl / t_coarse / 1e9 / PEAK_FP64_TFLOPS, 4),
                     "v_reorder_with_pooling_ms": round(t_vpool, 4)}
    sub, G = (2, 2, 2), 8
    qr = torch.empty((B, H, n * G, d), dtype=torch.float64, device=dev)
    kr = torch.empty_like(qr)
    rs = torch.empty((B, H, n, n), dtype=torch.float64, device=dev)
    t_rpool = time_call(lambda: (sa.sparse_attn_router_pool(path.qc, qr, g, sub),
                                 sa.sparse_attn_router_pool(path.kc, kr, g, sub)), reps)
    # the two passes that need no scratch, and one pass over the sub-cube scores
    # with its per-block sums in a workspace (the figures reported), each timed once
    ws64 = torch.empty(sa.sparse_attn_router_workspace_bytes(g, sub, 8), dtype=torch.uint8, device=dev)
    t_router2 = time_call(lambda: sa.sparse_attn_router_scores(qr, kr, rs, 0.0, g, sub), 1)
    t_router = time_call(lambda: sa.sparse_attn_router_scores(qr, kr, rs, 0.0, g, sub, ws64), 1)
    del ws64
    fl = 2.0 * B * H * (n * G) ** 2 * d              # one product per sub-cube score
    out["router_2x2x2"] = {"ms": round(t_router, 3), "pool_ms": round(t_rpool, 4),
                           "tflops_fp64": round(fl / t_router / 1e9, 2),
                           "frac_of_fp64_peak": round(fl / t_router / 1e9 / PEAK_FP64_TFLOPS, 4),
                           "two_pass_ms": round(t_router2, 3)}
    # the float32 router on the same means, and how many rows' lists differ from the float64 ones
    rs32 = torch.empty((B, H, n, n), dtype=torch.float32, device=dev)
    ws32 = torch.empty(sa.sparse_attn_router_workspace_bytes(g, sub, 4), dtype=torch.uint8, device=dev)
    t_r32b = time_call(lambda: sa.sparse_attn_router_scores_f32(qr, kr, rs32, 0.0, g, sub), 1)
    t_r32 = time_call(lambda: sa.sparse_attn_router_scores_f32(qr, kr, rs32, 0.0, g, sub, ws32), 1)
    del ws32
    la, ca = (torch.empty((B, H, n, n), dtype=torch.int32, device=dev), torch.empty((B, H, n), dtype=torch.int32,
                                                                                       device=dev))
    lb, cb = torch.empty_like(la), torch.empty_like(ca)
    sa.sparse_attn_select(rs, g, path.k_frac, path.p, None, la, ca, n)
    sa.sparse_attn_select_f32(rs32, g, path.k_frac, path.p, None, lb, cb, n)
    m = torch.arange(n, device=dev)[None, None, None, :] < ca[..., None]
    differ = int((~((ca == cb) & torch.where(m, la == lb, True).all(-1))).sum())
    out["router_2x2x2_f32"] = {"ms": round(t_r32, 3),
                               "tflops": round(fl / t_r32 / 1e9, 2),
                               "frac_of_fp32_matrix_peak": round(fl / t_r32 / 1e9 / PEAK_FP32_MFMA_TFLOPS, 4),
                               "two_pass_ms": round(t_r32b, 3),
                               "rows_differing_from_fp64_lists": differ, "rows": B * H * n}
    del qr, kr, rs, rs32, la, lb
    # backward over the same lists: the slot-major forward outputs and the
    # operand layouts it reads are prepared untimed
    sa.sparse_attn_fwd(path.qc, path.kc, path.vc, path.lut, path.counts, path.cap, g, 0.0, path.oc, path.lse_c,
                       path.fws)
    lay = {}
    for name, x, layout in (("q", path.q, sa.SA_LAYOUT_QK), ("k", path.k, sa.SA_LAYOUT_QK),
                            ("v_qk", path.v, sa.SA_LAYOUT_QK), ("k_v", path.k, sa.SA_LAYOUT_V),
                            ("do_qk", path.o_grad, sa.SA_LAYOUT_QK)):
        lay[name] = sa.reorder(x, g, layout)
    delta = torch.empty((B, H, path.n_pad), dtype=torch.float32, device=dev)
    lut_t = torch.empty((B, H, n, n), dtype=torch.int32, device=dev)
    counts_t = torch.empty((B, H, n), dtype=torch.int32, device=dev)
    ws = torch.empty(max(sa.sparse_attn_transpose_workspace_bytes(g), 256), dtype=torch.uint8, device=dev)
    dq, dk, dv = (torch.empty_like(path.oc) for _ in range(3))
    args = sa.BwdArgs(*(lay[k_].data_ptr() for k_ in ("q", "k", "v_qk", "k_v", "do_qk")),
                      path.lse_c.data_ptr(), delta.data_ptr(), path.lut.data_ptr(), path.counts.data_ptr(),
                      path.cap, lut_t.data_ptr(), counts_t.data_ptr(), n)
    t_delta = time_call(lambda: sa.sparse_attn_bwd_delta(path.oc, lay["do_qk"], delta, g), reps)
    t_tr = time_call(lambda: sa.sparse_attn_transpose_lut(path.lut, path.counts, path.cap, lut_t, counts_t, n, g,
                                                          ws), reps)
    t_bwd = time_call(lambda: sa.sparse_attn_bwd(args, g, 0.0, dq, dk, dv), reps)
    kept = int(path.counts.sum().item())
    fl = kept * 10.0 * 64 * 64 * d                    # five 64x64xd products per kept pair
    out["backward"] = {"ms": round(t_bwd, 4), "delta_ms": round(t_delta, 4), "transpose_ms": round(t_tr, 4),
                       "tflops": round(fl / t_bwd / 1e9, 2),
                       "frac_of_bf16_peak": round(fl / t_bwd / 1e9 / PEAK_BF16_TFLOPS, 4),
                       "flops_note": "10*64*64*d per kept block pair (the five products of the gradient)"}
    del lay, dq, dk, dv, lut_t
    # asymmetric blocks: query blocks of 2 cubes (128 query slots), one list each
    nq = -(-n // 2)
    lut2 = torch.empty((B, H, nq, n), dtype=torch.int32, device=dev)
    counts2 = torch.empty((B, H, nq), dtype=torch.int32, device=dev)
    ws2 = torch.empty(sa.sparse_attn_mask_groups_workspace_bytes(g, 2), dtype=torch.uint8, device=dev)
    t_m2 = time_call(lambda: sa.sparse_attn_build_mask_groups(path.qc, path.kc, g, 2, path.k_frac, path.p, lut2,
                                                              counts2, n, ws2), reps)
    oc2, lse2 = torch.empty_like(path.oc), torch.empty_like(path.lse_c)
    t_f2 = time_call(lambda: sa.sparse_attn_fwd_groups(path.qc, path.kc, path.vc, lut2, counts2, n, 2, g, 0.0,
                                                       oc2, lse2), reps)
    c2 = counts2.to(torch.int64)
    pairs = int(2 * c2.sum().item() - (c2[..., -1].sum().item() if n % 2 else 0))
    fl = pairs * 4.0 * 64 * 64 * d
    out["query_blocks_128"] = {"mask_ms": round(t_m2, 4), "fwd_ms": round(t_f2, 4),
                               "density": round(pairs / (B * H * n * n), 4),
                               "fwd_tflops": round(fl / t_f2 / 1e9, 2),
                               "frac_of_bf16_peak": round(fl / t_f2 / 1e9 / PEAK_BF16_TFLOPS, 4)}
    del lut2, oc2
    # per-sequence Top-K on the same block scores (one budget per head)
    lut3 = torch.empty((B, H, n, n), dtype=torch.int32, device=dev)
    counts3 = torch.empty((B, H, n), dtype=torch.int32, device=dev)
    ws3 = torch.empty(sa.sparse_attn_sequence_workspace_bytes(g), dtype=torch.uint8, device=dev)
    t_seq = time_call(lambda: sa.sparse_attn_select_per_sequence(path.scores, g, path.k_frac, lut3, counts3, n,
                                                                 ws3), reps)
    c3 = counts3.to(torch.float64)
    out["per_sequence_topk"] = {"ms": round(t_seq, 4), "budget_per_head": int(n * sa.sparse_attn_ceil_k(path.k_frac, n)),
                                "row_count_min": int(c3.min()), "row_count_max": int(c3.max()),
                                "rows_empty_frac": round(float((c3 == 0).to(torch.float64).mean()), 4)}
    del lut3
    # mask quality of the timed lists against dense attention (every block kept)
    t0 = time.perf_counter()
    mass, tau, rel = sa.mask_quality(path.qc, path.kc, path.vc, path.lut, path.counts, path.scores, g)
    torch.cuda.synchronize()
    real = tau > 0
    out["mask_quality"] = {"seconds": round(time.perf_counter() - t0, 3),
                           "mean_pooled_mass": round(float(mass.mean()), 5),
                           "mean_tau": round(float(tau[real].mean()), 5),
                           "min_tau": round(float(tau[real].min()), 5),
                           "mean_rel_l1": round(float(rel.mean()), 5)}
    del mass, tau, rel
    # ideal block scores (block-pooled full attention) and the recall of the timed lists
    full = torch.empty((B, H, n, n), dtype=torch.int32, device=dev)
    full_counts = torch.empty((B, H, n), dtype=torch.int32, device=dev)
    sa.sparse_attn_select(path.scores, g, 0.0, 1.0, None, full, full_counts, n)
    _, lse_d = sa.fwd(path.qc, path.kc, path.vc, full, full_counts, g)
    del full
    ideal = torch.empty((B, H, n, n), dtype=torch.float64, device=dev)
    t_ideal = time_call(lambda: sa.sparse_attn_ideal_block_mass(path.qc, path.kc, lse_d, g, 0.0, ideal), 1)
    recall = torch.empty((B, H, n), dtype=torch.float64, device=dev)
    ws_r = torch.empty(sa.sparse_attn_recall_workspace_bytes(g), dtype=torch.uint8, device=dev)
    t_rec = time_call(lambda: sa.sparse_attn_mask_recall(ideal, path.lut, path.counts, path.cap, g, recall, ws_r), 1)
    fl = 2.0 * B * H * (n * 64) ** 2 * d
    out["ideal_mass_recall"] = {"ideal_mass_ms": round(t_ideal, 3), "recall_ms": round(t_rec, 3),
                                "ideal_mass_tflops": round(fl / t_ideal / 1e9, 1),
                                "mean_recall": round(float(recall.mean()), 5)}
    return out


def machine_check(dev):
    """The box's own ceilings beside the published peaks: a plain 1 GiB
    device copy (HBM read + write) and a dense bf16 GEMM through the vendor
    library (torch.matmul), each event-timed."""
    x = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    t_copy = time_call(lambda: y.copy_(x), 10)
    m = 8192
    a = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    b = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    t_mm = time_call(lambda: torch.matmul(a, b), 10)
    del x, y, a, b
    return {"copy_gbps": round(2 * (1 << 30) / (t_copy * 1e-3) / 1e9, 1),
            "dense_bf16_gemm_tflops": round(2.0 * m ** 3 / (t_mm * 1e-3) / 1e12, 1),
            "note": "1 GiB device copy (bytes read + written); 8192^3 bf16 torch.matmul"}


def _oracle_worker(task):
    """One worker of the CPU baseline: the oracle's mask of one whole head,
    then its attention on the head's query blocks (in a seeded random order)
    until `seconds` have passed.  Returns (mask seconds, attention seconds,
    flops, query blocks done)."""
    wid, k_frac, p, budgets, h, seconds = task
    import oracle as O
    wl = synth.WORKLOADS[wid]
    og = O.Geometry(wl.frames, wl.height, wl.width)
    q, k, v = synth.head_qkv(wl, 0, h, 0)
    qc, kc, vc = (O.reorder(t.double().numpy(), og) for t in (q, k, v))
    t0 = time.perf_counter()
    s = O.block_scores(O.pool(qc, og), O.pool(kc, og), wl.head_dim)
    if budgets:
        rb = synth.row_budgets(wl, 0)[0, h]
        probs = O.block_softmax(s)
        sels = [O.select_row(s[i], int(rb[i]), 0.0, probs[i]) for i in range(og.nblk)]
    else:
        sels = O.select_rows(s, O.ceil_k(k_frac, og.nblk), p)
    t_mask = time.perf_counter() - t0
    # the oracle's report of this head's mask (outside the timed parts)
    counts = np.array([[[x.kept.size for x in sels]]])
    density, sink, entropy = (float(a[0, 0]) for a in O.mask_report(s[None, None], counts))
    report = (wl.head_types[h], density, sink, entropy)
    flops, done = 0.0, 0
    t1 = time.perf_counter()
    for i in np.random.default_rng(h).permutation(og.nblk):
        O.attention_block(qc, kc, vc, sels[i].kept, og, int(i))
        flops += sels[i].kept.size * 4.0 * 64 * 64 * wl.head_dim
        done += 1
        if time.perf_counter() - t1 > seconds:
            break
    return t_mask, time.perf_counter() - t1, flops, done, report


def cpu_baseline(wl, seconds, workload, workers=16):
    """The oracle, as it stands, on a bounded sample of the same workload, on
    `workers` host processes with one BLAS thread each: one whole head per
    worker (its mask, then the attention of its query blocks for at most
    `seconds`); value = oracle flops on kept blocks / the slowest worker's
    compute time."""
    import concurrent.futures as cf
    import multiprocessing as mp
    wid, k_frac, p, budgets = WORKLOADS[workload]
    heads = list(range(min(workers, wl.heads)))
    tasks = [(wid, k_frac, p, budgets, h, seconds) for h in heads]
    env_keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in env_keys}
    for k in env_keys:
        os.environ[k] = "1"            # one thread per worker process
    try:
        t0 = time.perf_counter()
        with cf.ProcessPoolExecutor(max_workers=len(tasks), mp_context=mp.get_context("spawn")) as ex:
            res = list(ex.map(_oracle_worker, tasks))
        wall = time.perf_counter() - t0
    finally:
        for k, val in saved.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val
    flops = sum(r[2] for r in res)
    done = sum(r[3] for r in res)
    busy = max(r[0] + r[1] for r in res)    # the slowest worker (process start-up excluded)
    # the oracle's mask report of the sampled heads, by head type: realised
    # block density, mean sink mass (probability on block 0) and mean row
    # entropy of the block softmax (ln nblk for a flat row)
    by_type = {}
    for r in res:
        kind, density, sink, entropy = r[4]
        by_type.setdefault(kind, []).append((density, sink, entropy))
    mask_report = {kind: {"heads": len(v), "density": round(float(np.mean([x[0] for x in v])), 5),
                          "sink_mass": round(float(np.mean([x[1] for x in v])), 5),
                          "row_entropy": round(float(np.mean([x[2] for x in v])), 4),
                          "ln_nblk": round(math.log(wl.n_blocks()), 4)}
                   for kind, v in sorted(by_type.items())}
    return {
        "value": flops / busy / 1e12,
        "unit": "TFLOPS",
        "cores": len(tasks),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle on {len(tasks)} processes of one thread each, one whole head "
                   f"per process: the mask of {len(heads)} heads (pool, scores, selection of every row; "
                   f"{max(r[0] for r in res):.2f}s at most) and the attention of {done} of their "
                   f"{len(heads) * wl.n_blocks()} query blocks (at most {seconds:.0f}s per "
                   f"process); value = kept-block flops / the slowest process's time"),
        "seconds": round(busy, 2),
        "wall_seconds_with_startup": round(wall, 2),
        "oracle_mask_report": mask_report,
        "host_cpus": os.cpu_count(),
        "cpu_model": cpu_model(),
    }


def other_workloads(dev, names, reps=3):
    """The forward as the whole-path call runs it (token order; the
    count-balanced row order with per-row budgets) on the other workloads,
    each on freshly generated inputs and its GPU-built lists: time, kept-block
    TFLOP/s and fraction of the bf16 peak.  Not part of `value`."""
    out = {}
    for name in names:
        wid, k_frac, p, budgets = WORKLOADS[name]
        wl = synth.WORKLOADS[wid]
        g = sa.make_geom(wl.batch, wl.heads, wl.frames, wl.height, wl.width, wl.head_dim)
        nblk, n_real, _ = sa.sparse_attn_geometry(g)
        q, k, v = synth.make_qkv(wl, 0)
        qc = sa.reorder(q.to(dev), g, sa.SA_LAYOUT_QK)
        kc = sa.reorder(k.to(dev), g, sa.SA_LAYOUT_QK)
        vc = sa.reorder(v.to(dev), g, sa.SA_LAYOUT_V)
        del q, k, v
        rb = torch.from_numpy(synth.row_budgets(wl, 0)).to(dev) if budgets else None
        lut, counts = sa.build_mask(qc, kc, g, k_frac, p, row_budget=rb)
        o = torch.empty((wl.batch, wl.heads, n_real, wl.head_dim), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((wl.batch, wl.heads, n_real), dtype=torch.float32, device=dev)
        ws = torch.empty(sa.sparse_attn_fwd_workspace_bytes(g), dtype=torch.uint8, device=dev) if budgets else None
        ms = time_call(lambda: sa.sparse_attn_fwd_tokens(qc, kc, vc, lut, counts, nblk, g, 0.0, o, lse, ws), reps)
        kept = int(counts.sum().item())
        tf = kept * 4.0 * 64 * 64 * wl.head_dim / (ms * 1e-3) / 1e12
        out[name] = {"fwd_ms": round(ms, 3), "fwd_tflops": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                     "block_sparsity": round(1.0 - kept / (wl.batch * wl.heads * nblk * nblk), 5),
                     "kept_blocks": kept, "heads": wl.heads, "k_frac": k_frac, "p": p, "row_budgets": budgets}
        log(f"[bench] {name}: fwd {ms:.3f} ms, {tf:.1f} TFLOP/s")
        del qc, kc, vc, lut, counts, o, lse
        torch.cuda.empty_cache()
    return out


def cpu_model():
    """The host CPU's model name, as /proc/cpuinfo gives it (None elsewhere)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        log("bench.py: only --gpus 1 is supported (the path runs on one GPU; it would shard by "
            "(batch, head), with no exchange inside the attention)")
        sys.exit(2)
    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    dev = torch.device("cuda:0")
    wid, k_frac, p, budgets = WORKLOADS[args.workload]
    wl = synth.WORKLOADS[wid]
    path = Path(wl, k_frac, p, budgets, dev)
    log(f"[bench] {args.workload}: {path.g}, nblk={path.nblk}, k_frac={k_frac}, p={p}")

    step = path.step if args.serial else (lambda: path.step_call(args.overlap))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # per-stage breakdown: the same kernels one after another, event-timed
    names = [n for n, _ in path.stages()]
    nst = max(3, min(args.steps, 10))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(nst)]
    torch.cuda.synchronize()
    for s_ in range(nst):
        ev[s_][0].record()
        for j, (_, fn) in enumerate(path.stages()):
            fn()
            ev[s_][j + 1].record()
    torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([ev[s_][j].elapsed_time(ev[s_][j + 1]) for s_ in range(nst)]))
                for j, n in enumerate(names)}

    kept = int(path.counts.sum().item())
    rows = wl.batch * wl.heads * path.nblk
    density = kept / (rows * path.nblk)
    flops_kept = kept * 4.0 * 64 * 64 * wl.head_dim
    flops_real = 4.0 * path.n_real ** 2 * wl.head_dim * wl.heads * wl.batch * density
    value = flops_kept / (ms_per_step * 1e-3) / 1e12
    fwd_tflops = flops_kept / (stage_ms["fwd"] * 1e-3) / 1e12
    abytes = algorithmic_bytes(path)
    gbps = {n: abytes[n] / (stage_ms[n] * 1e-3) / 1e9 for n in abytes}
    mask_path_gbps = (abytes["reorder"] + abytes["mask"]) / (
        (stage_ms["reorder"] + stage_ms["mask"]) * 1e-3) / 1e9
    mbytes = min_bytes(path)
    mask_path_gbps_min = (mbytes["reorder"] + mbytes["mask"]) / (
        (stage_ms["reorder"] + stage_ms["mask"]) * 1e-3) / 1e9

    # the mask phase as the library runs it: sparse_attn_mask_path on two
    # streams (re-indexing on one beside the scores and selection on the other)
    t_mask_ov = time_call(lambda: sa.sparse_attn_mask_path(path.buf, path.g, path.k_frac, path.p,
                                                           aux_stream=path.aux.cuda_stream), 10)
    mask_overlapped = {
        "ms": round(t_mask_ov, 4),
        "gbps_min_bytes": round((mbytes["reorder"] + mbytes["mask"]) / (t_mask_ov * 1e-3) / 1e9, 1),
        "min_bytes_frac_of_hbm": round((mbytes["reorder"] + mbytes["mask"]) / (t_mask_ov * 1e-3) / 1e9
                                       / PEAK_HBM_GBPS, 4),
        "gbps_implementation_bytes": round((abytes["reorder"] + abytes["mask"]) / (t_mask_ov * 1e-3) / 1e9, 1),
        "note": ("sparse_attn_mask_path with an auxiliary stream: rows in 4 parts, each part's scores and "
                 "selection beside the next parts' re-indexing; event-timed on the calling stream"),
    }

    if args.copy_calibration:
        # a 1 GiB device copy and a 1 GiB elementwise kernel (y = x * 1), each
        # reading and writing 1 GiB: counter calibration
        x = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        xf, yf = x.view(torch.float32), y.view(torch.float32)
        for _ in range(3):
            torch.mul(xf, 1.0, out=yf)
        torch.cuda.synchronize()
        del x, y, xf, yf

    out = {
        "metric": "sparse-attn effective TFLOPS @95% sparsity, 75.6K tok; % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Wan2.1-720p-shaped Q/K/V, uniform/skewed/local heads)",
        "config": {
            "workload": (f"{args.workload}: B={wl.batch} H={wl.heads} d={wl.head_dim} grid "
                         f"{wl.frames}x{wl.height}x{wl.width} ({path.n_real} tokens, {path.nblk} "
                         f"blocks of 64), k_frac={k_frac}, p={p}"),
            "global_batch": wl.batch,
            "seq_len": path.n_real,
            "parallelism": "single GPU",
            "schedule": ("stages launched from Python on one stream" if args.serial else
                         "sparse_attn_attention on one stream" if args.overlap == 0 else
                         "sparse_attn_attention on two streams: re-indexing of one half of the heads "
                         "(and of the values) beside the scores and selection of the other" if args.overlap < 0 else
                         f"sparse_attn_attention, mask of chunk c+1 beside forward of chunk c "
                         f"({args.overlap} rows per chunk, two streams)"),
            "block_sparsity": round(1.0 - density, 5),
            "kept_blocks": kept,
        },
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_tflops, 2),
        "real_token_tflops": round(flops_real / (ms_per_step * 1e-3) / 1e12, 2),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stage_gbps": {k: round(v, 1) for k, v in gbps.items()},
        "mask_path_gbps": round(mask_path_gbps, 1),
        "mask_path_frac_of_hbm": round(mask_path_gbps / PEAK_HBM_GBPS, 4),
        "mask_path_gbps_min_bytes": round(mask_path_gbps_min, 1),
        "mask_path_min_bytes_frac_of_hbm": round(mask_path_gbps_min / PEAK_HBM_GBPS, 4),
        "mask_path_overlapped": mask_overlapped,
        "mask_path_bytes": {"implementation": int(abytes["reorder"] + abytes["mask"]),
                            "minimum": int(mbytes["reorder"] + mbytes["mask"]),
                            "note": ("implementation: float64 means and float32 scores as this library keeps "
                                     "them; minimum: Q/K/V read and written once, scores float32 written and "
                                     "read once, lists written once")},
        "roofline": {
            "bound": "mfma",
            "achieved": round(fwd_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": recorded_traffic(args.workload),
        },
    }
    if not args.no_next_rows:
        log("[bench] timing the coarse-output and router kernels")
        out["next_rows"] = next_rows(path)
        out["machine_check"] = machine_check(dev)
    if not args.no_other_workloads:
        del path
        torch.cuda.empty_cache()
        log("[bench] timing the forward on the other workloads")
        out["other_workloads"] = other_workloads(dev, [w for w in WORKLOADS if w != args.workload])
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, args.workload)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
