"""The allocation-free mask entry point (sparse_attn_build_mask_noalloc) against
sparse_attn_build_mask with a caller workspace, through the C ABI: the same
lists and counts, bit for bit, on calls in a row with different shapes (the
library's scratch array keeps the previous call's contents)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_hybrid_amd as sa
import synth
from _helpers import geom_of, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(wl, seed=0, heads=None):
    q, k, _ = synth.make_qkv(wl, seed, heads=heads)
    nh = wl.heads if heads is None else len(heads)
    g = sa.make_geom(wl.batch, nh, wl.frames, wl.height, wl.width, wl.head_dim)
    qc = sa.reorder(q.to(DEV), g, sa.SA_LAYOUT_QK)
    kc = sa.reorder(k.to(DEV), g, sa.SA_LAYOUT_QK)
    return g, qc, kc


def _both(g, qc, kc, k_frac, p, budget=None):
    nblk = sa.sparse_attn_geometry(g)[0]
    shape = (g.batch, g.heads, nblk)
    rb = None if budget is None else torch.from_numpy(budget).to(DEV)
    lut_a = torch.full(shape + (nblk,), -3, dtype=torch.int32, device=DEV)
    cnt_a = torch.full(shape, -3, dtype=torch.int32, device=DEV)
    sa.sparse_attn_build_mask_noalloc(qc, kc, g, 64, k_frac, p, rb, lut_a, cnt_a, nblk)
    ws = torch.empty(sa.sparse_attn_mask_workspace_bytes(g), dtype=torch.uint8, device=DEV)
    lut_b = torch.full(shape + (nblk,), -3, dtype=torch.int32, device=DEV)
    cnt_b = torch.full(shape, -3, dtype=torch.int32, device=DEV)
    sa.sparse_attn_build_mask(qc, kc, g, 64, k_frac, p, rb, lut_b, cnt_b, nblk, ws)
    torch.cuda.synchronize()
    assert torch.equal(cnt_a, cnt_b)
    live = torch.arange(nblk, device=DEV) < cnt_a[..., None]
    assert torch.equal(torch.where(live, lut_a, 0), torch.where(live, lut_b, 0))
    return cnt_a


def test_noalloc_mask_equals_workspace_mask_on_calls_in_a_row():
    scratch = sa.sparse_attn_build_mask_noalloc_scratch_bytes()
    # 720p shape, 4 heads: about 19.5 MB of means and scores per head, so the
    # 64 MiB array takes the rows in two chunks (3 + 1)
    wl = synth.WORKLOADS[2]
    say(f"[no-alloc] 720p, 4 heads (scratch {scratch >> 20} MiB)")
    g, qc, kc = _inputs(wl, heads=[0, 1, 2, 3])
    cnt = _both(g, qc, kc, 0.03, 0.073)
    say(f"  720p lists identical; density {cnt.double().mean().item() / 1440:.4f}")
    # then a smaller call (batch 2, ragged grid) and a row-budget call
    wl2 = synth.custom_workload(2, 3, 128, 5, 7, 9)
    g2, qc2, kc2 = _inputs(wl2, seed=1)
    _both(g2, qc2, kc2, 0.3, 0.6)
    nblk2 = sa.sparse_attn_geometry(g2)[0]
    budget = np.random.default_rng(2).integers(0, nblk2 + 1, size=(2, 3, nblk2)).astype(np.int32)
    _both(g2, qc2, kc2, 0.0, 0.0, budget)
    say("  small ragged and row-budget calls identical")
