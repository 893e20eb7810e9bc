"""Parity at the full workload sizes, in the launch configuration the benchmark
times: the whole path runs on the GPU for every head; the oracle recomputes
every head's kept-block lists and the attention of sampled query blocks (every
query block of one head, and the longest-list tenth of the others, on the
sparsest workloads), with its own lists fed to the GPU attention; properties
that hold at any size are checked on every row."""
import functools
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_hybrid_amd as sa
import oracle as O
import synth
from _helpers import (LSE_MAX_ABS, LSE_MEAN_ABS, O_MAX_ABS, O_MEAN_ABS, attn_errors,
                      compare_lists, geom_of, grad_errors, lse_errors, ogeom_of, say, to64)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda:0"

# name, workload id, k_frac, p, row budgets, sampled heads, every row of the
# first sampled head (plus the longest-list tenth of the others) checked
CASES = [
    ("480p", 1, 0.05, 0.9, False, (0, 1, 2), False),
    ("720p-literal", 2, 0.03, 0.85, False, (0, 1, 2), False),
    ("720p-hybrid95", 2, 0.03, 0.073, False, (0, 1, 2, 39), True),
    ("720p-extreme", 3, 0.02, 0.8, False, (0, 7, 20, 22), False),
    ("720p-97", 3, 0.02, 0.052, False, (0, 7, 20, 22), True),
    ("720p-varbudget", 4, 0.0, 0.0, True, (0, 1, 2), True),
]


@pytest.mark.parametrize("name,wid,k_frac,p,budgets,heads,all_rows", CASES, ids=[c[0] for c in CASES])
def test_workload(name, wid, k_frac, p, budgets, heads, all_rows):
    wl = synth.WORKLOADS[wid]
    say(f"[workload {name}] H={wl.heads} d={wl.head_dim} grid={wl.grid} k={k_frac} p={p}")
    g, og = geom_of(wl), ogeom_of(wl)
    n = og.nblk
    q, k, v = synth.make_qkv(wl, 0)
    rb_np = synth.row_budgets(wl, 0) if budgets else None
    rb = torch.from_numpy(rb_np).to(DEV) if budgets else None
    qc = sa.reorder(q.to(DEV), g, sa.SA_LAYOUT_QK)
    kc = sa.reorder(k.to(DEV), g, sa.SA_LAYOUT_QK)
    vc = sa.reorder(v.to(DEV), g, sa.SA_LAYOUT_V)
    lut, counts = sa.build_mask(qc, kc, g, k_frac, p, row_budget=rb)
    oc, lse_c = sa.fwd(qc, kc, vc, lut, counts, g)
    torch.cuda.synchronize()
    say("  gpu path done")

    # --- properties on every row --------------------------------------------
    counts_h = counts.cpu().numpy()
    kc_all = rb_np if budgets else np.full_like(counts_h, O.ceil_k(k_frac, n))
    assert np.all(counts_h >= np.minimum(kc_all, n)) and np.all(counts_h <= n)
    if budgets:
        assert np.array_equal(counts_h, np.clip(rb_np, 0, n))
    lut_h = lut.cpu().numpy()
    pos = np.arange(n)[None, None, None, :]
    live = pos < counts_h[..., None]
    ids = np.where(live, lut_h, -1)
    assert np.all(ids[live] >= 0) and np.all(ids[live] < n)
    inc = np.diff(np.where(live, lut_h, n + pos), axis=-1)
    assert np.all(inc > 0), "kept ids must be strictly ascending"
    real = O.real_slots(og)
    lse_h = lse_c.cpu().numpy()
    assert np.all(np.isfinite(lse_h[..., real])) and np.all(np.isneginf(lse_h[..., ~real]))
    assert bool(torch.isfinite(oc).all())
    density = counts_h.sum() / (counts_h.size * n)
    say(f"  density {density:.4f} (block sparsity {1 - density:.4f})")

    # --- the configuration the bench times: the whole-path call on two streams,
    # all rows in one chunk, O and LSE straight to token order.  Same lists, and
    # the same bytes as the checked step-by-step path re-indexed.
    o_ref_path, lse_ref_path = sa.unreorder(oc, lse_c, g)
    buf, t = sa.path_buffers(q.to(DEV), k.to(DEV), v.to(DEV), g, row_budget=rb, slot_major=False)
    aux = torch.cuda.Stream()
    sa.sparse_attn_attention(buf, g, k_frac, p, 0.0, g.batch * g.heads, aux_stream=aux.cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(t["counts"], counts)
    live_t = torch.arange(n, device=DEV) < counts[..., None]
    assert torch.equal(torch.where(live_t, t["lut"], 0), torch.where(live_t, lut, 0))
    assert torch.equal(t["o"], o_ref_path) and torch.equal(t["lse"], lse_ref_path)
    del buf, t, o_ref_path, lse_ref_path
    say("  whole-path call (bench configuration) identical")

    # the float32 block scores the path selects on, from its own means
    qbar = torch.empty((wl.batch, wl.heads, n, wl.head_dim), dtype=torch.float64, device=DEV)
    kbar = torch.empty_like(qbar)
    sa.sparse_attn_pool(qc, kc, qbar, kbar, g)
    s32 = torch.empty((wl.batch, wl.heads, n, n), dtype=torch.float32, device=DEV)
    sa.sparse_attn_block_scores_f32(qbar, kbar, s32, 0.0, g)
    s32_h = s32.cpu().numpy()
    del qbar, kbar, s32

    # --- oracle lists on every head (one head at a time) ---------------------
    sel = list(heads)
    refs = {}
    n_bad = n_near = n_invalid = 0
    worst_score = 0.0
    for h in range(wl.heads):
        qs, ks = (O.reorder(to64(t[:, h:h + 1]), og) for t in (q, k))
        ref = O.build_mask(qs, ks, og, k_frac, p, row_budget=None if not budgets else rb_np[:, h:h + 1])
        # scores within 5e-7 of each row's largest |score|: a pair of scores
        # at least the 1e-6 near-tie margin apart keeps its order
        rowmax = np.abs(ref.scores[0, 0]).max(axis=-1, keepdims=True)
        err = float((np.abs(s32_h[0, h].astype(np.float64) - ref.scores[0, 0]) / rowmax).max())
        worst_score = max(worst_score, err)
        assert err <= 5e-7, (h, err)
        bad, near, invalid = compare_lists(lut_h[:, h:h + 1], counts_h[:, h:h + 1], ref, p)
        n_bad, n_near, n_invalid = n_bad + len(bad), n_near + near, n_invalid + len(invalid)
        assert not bad and not invalid, (h, bad[:4], invalid[:4])
        if h in sel:
            refs[h] = ref
    say(f"  lists on all {wl.heads} heads: {n_bad} mismatches outside near ties, {n_near} near ties, "
        f"{n_invalid} invalid; float32 scores within {worst_score:.2e} of each row's largest |score|")

    # oracle lists fed to the GPU attention, on the sampled heads at full shape
    ref_lut = np.concatenate([refs[h].lut for h in sel], axis=1)
    ref_counts = np.concatenate([refs[h].counts for h in sel], axis=1)
    gs = sa.make_geom(wl.batch, len(sel), wl.frames, wl.height, wl.width, wl.head_dim)
    qcs, kcs, vcs = (x[:, sel].contiguous() for x in (qc, kc, vc))
    ocs, lses = sa.fwd(qcs, kcs, vcs, torch.from_numpy(ref_lut).to(DEV), torch.from_numpy(ref_counts).to(DEV), gs)
    torch.cuda.synchronize()
    ocs_h, lses_h = to64(ocs), lses.cpu().double().numpy()
    qs, ks, vs = (O.reorder(to64(t[:, sel]), og) for t in (q, k, v))
    rng = np.random.default_rng(1)
    base_rows = sorted(set([0, 1, n // 2, n - 1] + list(rng.integers(0, n, 4))))
    worst = [0.0, 0.0, 0.0, 0.0]
    checked = 0
    for hi in range(len(sel)):
        rows = set(base_rows)
        if all_rows:
            c = ref_counts[0, hi]
            rows |= set(np.argsort(-c, kind="stable")[:max(1, n // 10)].tolist())   # longest lists
            if hi == 0:
                rows = set(range(n))
        for i in sorted(rows):
            kept = ref_lut[0, hi, i, :ref_counts[0, hi, i]]
            o_ref, l_ref = O.attention_block(qs[0, hi], ks[0, hi], vs[0, hi], kept, og, i)
            blk_real = real[i * 64:(i + 1) * 64]
            mx, mean = attn_errors(ocs_h[0, hi, i * 64:(i + 1) * 64], o_ref, blk_real)
            lmx, lmean = lse_errors(lses_h[0, hi, i * 64:(i + 1) * 64], l_ref)
            worst = [max(worst[0], mx), max(worst[1], mean), max(worst[2], lmx), max(worst[3], lmean)]
            assert mx <= O_MAX_ABS and mean <= O_MEAN_ABS, (sel[hi], i, mx, mean)
            assert lmx <= LSE_MAX_ABS and lmean <= LSE_MEAN_ABS, (sel[hi], i, lmx, lmean)
            assert not np.any(ocs_h[0, hi, i * 64:(i + 1) * 64][~blk_real])
            checked += 1
            # where the lists agree, the main run's output is the same computation
            if counts_h[0, sel[hi], i] == kept.size and np.array_equal(lut_h[0, sel[hi], i, :kept.size], kept):
                main = to64(oc[0, sel[hi], i * 64:(i + 1) * 64])
                assert np.array_equal(main, ocs_h[0, hi, i * 64:(i + 1) * 64])
    say(f"  attention on {checked} query blocks (real slots): O max {worst[0]:.2e} mean {worst[1]:.2e}; "
        f"LSE max {worst[2]:.2e} mean {worst[3]:.2e}")


@functools.lru_cache(maxsize=1)
def _router_720p_oracle():
    """The float64 oracle's router scores of two 720p heads (a uniform and a
    skewed one), 2x2x2 sub-cubes."""
    wl = synth.WORKLOADS[2]
    heads = [0, 1]
    q, k, _ = synth.make_qkv(wl, 0, heads=heads)
    og = ogeom_of(wl)
    ref_qc, ref_kc = O.reorder(to64(q), og), O.reorder(to64(k), og)
    want = np.stack([O.router_scores(ref_qc[0, h], ref_kc[0, h], og) for h in range(len(heads))])[None]
    return q, k, want


@pytest.mark.parametrize("one_pass", [True, False], ids=["one-pass", "two-pass"])
@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_router_full_size(dtype, one_pass):
    """Fine-grained router (2x2x2 sub-cubes, G = 8) at the 720p shape on two
    heads (a uniform and a skewed one): scores and kept lists against the
    oracle, in float64 and in float32, in one pass and in two."""
    wl = synth.WORKLOADS[2]
    say(f"[router 720p] {dtype}, {'one pass' if one_pass else 'two passes'}, grid={wl.grid}")
    q, k, want = _router_720p_oracle()
    g = sa.make_geom(1, 2, wl.frames, wl.height, wl.width, wl.head_dim)
    og = ogeom_of(wl)
    qc, kc = sa.reorder(q.to(DEV), g, sa.SA_LAYOUT_QK), sa.reorder(k.to(DEV), g, sa.SA_LAYOUT_QK)
    lut, counts, scores = sa.router_mask(qc, kc, g, 0.03, 0.073,
                                         dtype=torch.float32 if dtype == "f32" else torch.float64,
                                         one_pass=one_pass)
    torch.cuda.synchronize()
    say(f"  gpu router ({dtype}) done")
    got = scores.cpu().numpy().astype(np.float64)
    if dtype == "f32":
        rel = np.abs(got - want) / np.abs(want).max(axis=-1, keepdims=True)
        say(f"  router f32: max error {rel.max():.2e} of the row's largest |log P_r|")
        assert rel.max() <= 5e-6
    else:
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-11)
    from test_gpu_parity import _ref_lists
    ref = _ref_lists(want, O.ceil_k(0.03, og.nblk), 0.073)
    bad, near, invalid = compare_lists(lut.cpu().numpy(), counts.cpu().numpy(), ref, 0.073)
    density = counts.cpu().numpy().sum() / (counts.numel() * og.nblk)
    say(f"  router lists: {len(bad)} mismatches outside near ties, {near} near ties, density {density:.4f}")
    assert not bad and not invalid


def test_backward_full_size():
    """Backward at the 720p shape with the hybrid-95 mask on two heads; the
    float64 oracle recomputes head 0's gradients in full."""
    wl = synth.WORKLOADS[2]
    heads = [0, 1]
    say(f"[backward 720p] heads {heads}")
    q, k, v = synth.make_qkv(wl, 0, heads=heads)
    g = sa.make_geom(1, len(heads), wl.frames, wl.height, wl.width, wl.head_dim)
    og = ogeom_of(wl)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse, lut, counts = sa.attention(qd, kd, vd, g, 0.03, 0.073)
    qc, kc, vc = (sa.reorder(x, g, lay) for x, lay in ((qd, sa.SA_LAYOUT_QK), (kd, sa.SA_LAYOUT_QK),
                                                       (vd, sa.SA_LAYOUT_V)))
    oc, lse_c = sa.fwd(qc, kc, vc, lut, counts, g)
    rng = np.random.default_rng(5)
    do = torch.from_numpy(rng.standard_normal(tuple(q.shape)).astype(np.float32)).to(torch.bfloat16)
    dq, dk, dv = sa.backward(qd, kd, vd, do.to(DEV), oc, lse_c, lut, counts, g)
    torch.cuda.synchronize()
    say("  gpu backward done")
    h = 0
    ref_q, ref_k, ref_v, ref_do = (O.reorder(to64(x[:, h:h + 1]), og) for x in (q, k, v, do))
    want = O.sparse_attention_backward(ref_q, ref_k, ref_v, ref_do, lut[:, h:h + 1].cpu().numpy(),
                                       counts[:, h:h + 1].cpu().numpy(), og)
    real = O.real_slots(og)
    for got, w, name in zip((dq, dk, dv), want, ("dq", "dk", "dv")):
        emax, emean, scale = grad_errors(to64(got[:, h:h + 1]), w, real)
        say(f"  {name}: max err {emax:.2e} mean {emean:.2e} (real slots; max |grad| {scale:.2e})")
        assert emax <= 2e-2 * scale and emean <= 2e-3 * scale, name


def test_grouped_blocks_full_size():
    """Query blocks of 2 cubes (128 query slots) against single-cube key blocks
    at the 720p shape on two heads: every list against the oracle, and the
    forward of sampled query blocks on the GPU's lists."""
    wl = synth.WORKLOADS[2]
    heads = [0, 1]
    say(f"[groups 720p] heads {heads} grid={wl.grid}")
    q, k, v = synth.make_qkv(wl, 0, heads=heads)
    g = sa.make_geom(1, len(heads), wl.frames, wl.height, wl.width, wl.head_dim)
    og = ogeom_of(wl)
    qc, kc = sa.reorder(q.to(DEV), g, sa.SA_LAYOUT_QK), sa.reorder(k.to(DEV), g, sa.SA_LAYOUT_QK)
    vc = sa.reorder(v.to(DEV), g, sa.SA_LAYOUT_V)
    lut, counts = sa.build_mask_groups(qc, kc, g, 2, 0.03, 0.073)
    oc, lse_c = sa.fwd_groups(qc, kc, vc, lut, counts, g, 2)
    torch.cuda.synchronize()
    say("  gpu groups done")
    ref_qc, ref_kc, ref_vc = (O.reorder(to64(t), og) for t in (q, k, v))
    ref = O.build_mask_groups(ref_qc, ref_kc, og, 2, 0.03, 0.073)
    lut_h, counts_h = lut.cpu().numpy(), counts.cpu().numpy()
    bad, near, invalid = compare_lists(lut_h, counts_h, ref, 0.073)
    say(f"  group lists: {len(bad)} mismatches outside near ties, {near} near ties")
    assert not bad and not invalid
    rng = np.random.default_rng(5)
    oc_h, lse_h = to64(oc), lse_c.cpu().numpy().astype(np.float64)
    for h in range(len(heads)):
        for i in rng.choice(og.nblk, 12, replace=False):
            a = i // 2
            kept = lut_h[0, h, a, :counts_h[0, h, a]]
            o_ref, lse_ref = O.attention_block(ref_qc[0, h], ref_kc[0, h], ref_vc[0, h], kept, og, int(i))
            sl = slice(64 * i, 64 * i + 64)
            mx, mean = attn_errors(oc_h[0, h, sl], o_ref, O.real_slots(og)[sl])
            lmx, _ = lse_errors(lse_h[0, h, sl], lse_ref)
            assert mx <= O_MAX_ABS and mean <= O_MEAN_ABS and lmx <= LSE_MAX_ABS, (h, i, mx, mean, lmx)


def test_per_sequence_full_size():
    """Per-sequence Top-K at the 720p shape on three heads (one of each type),
    on the GPU's own block scores."""
    wl = synth.WORKLOADS[2]
    heads = [0, 1, 2]
    say(f"[per-sequence 720p] heads {heads}")
    q, k, _ = synth.make_qkv(wl, 0, heads=heads)
    g = sa.make_geom(1, len(heads), wl.frames, wl.height, wl.width, wl.head_dim)
    qc, qbar = sa.reorder_pool(q.to(DEV), g)
    kc, kbar = sa.reorder_pool(k.to(DEV), g)
    n = sa.sparse_attn_geometry(g)[0]
    s = torch.empty((1, len(heads), n, n), dtype=torch.float64, device=DEV)
    sa.sparse_attn_block_scores(qbar, kbar, s, 1.0 / math.sqrt(wl.head_dim), g)
    lut, counts = sa.select_per_sequence(s, g, 0.03)
    torch.cuda.synchronize()
    from test_gpu_parity import check_per_sequence
    c = counts.cpu().numpy()
    bad, near = check_per_sequence(lut.cpu().numpy(), c, s.cpu().numpy(), 0.03)
    say(f"  per-sequence: {bad} count mismatches, {near} near-tie rows; counts min {c.min()} max {c.max()}")
    assert bad == 0


@pytest.mark.parametrize("p", [0.1, 0.999], ids=["one-wave", "dense-groups"])
def test_largest_head(p):
    """The whole path at the largest head the library takes (4,096 blocks:
    a 16x128x128 latent grid, 262,144 tokens, one skewed head, d = 128), on
    lists of about a tenth of the blocks (the one-wave forward) and on nearly
    dense ones (the dense-group kernel, whose LDS list bitmaps are sized for
    4,096 blocks): every row's list against the
    oracle's, and the attention of sampled query blocks with the oracle's
    lists fed to the GPU forward."""
    wl = synth.custom_workload(1, 1, 128, 16, 128, 128, head_types=("skewed",), wid=101, name="largest")
    g, og = geom_of(wl), ogeom_of(wl)
    n = og.nblk
    assert n == 4096 and sa.sparse_attn_geometry(g)[0] == n
    say(f"[largest head] nblk={n} tokens={og.n_real} p={p}")
    q, k, v = synth.make_qkv(wl, 0)
    qc = sa.reorder(q.to(DEV), g, sa.SA_LAYOUT_QK)
    kc = sa.reorder(k.to(DEV), g, sa.SA_LAYOUT_QK)
    vc = sa.reorder(v.to(DEV), g, sa.SA_LAYOUT_V)
    lut, counts = sa.build_mask(qc, kc, g, 0.03, p)
    torch.cuda.synchronize()
    qs, ks, vs = (O.reorder(to64(t), og) for t in (q, k, v))
    ref = O.build_mask(qs, ks, og, 0.03, p)
    bad, near, invalid = compare_lists(lut.cpu().numpy(), counts.cpu().numpy(), ref, p)
    say(f"  lists: {len(bad)} mismatches outside near ties, {near} near ties, {len(invalid)} invalid; "
        f"mean count {ref.counts.mean():.1f}")
    assert not bad and not invalid
    oc, lse_c = sa.fwd(qc, kc, vc, torch.from_numpy(ref.lut).to(DEV), torch.from_numpy(ref.counts).to(DEV), g)
    torch.cuda.synchronize()
    oc_h, lse_h = to64(oc), lse_c.cpu().double().numpy()
    real = O.real_slots(og)
    for i in (0, 1, n // 2, n - 1):
        kept = ref.lut[0, 0, i, :ref.counts[0, 0, i]]
        o_ref, l_ref = O.attention_block(qs[0, 0], ks[0, 0], vs[0, 0], kept, og, i)
        mx, mean = attn_errors(oc_h[0, 0, i * 64:(i + 1) * 64], o_ref, real[i * 64:(i + 1) * 64])
        lmx, lmean = lse_errors(lse_h[0, 0, i * 64:(i + 1) * 64], l_ref)
        assert mx <= O_MAX_ABS and mean <= O_MEAN_ABS, (i, mx, mean)
        assert lmx <= LSE_MAX_ABS and lmean <= LSE_MEAN_ABS, (i, lmx, lmean)
    say(f"  attention of 4 query blocks within the bars")
