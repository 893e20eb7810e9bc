"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/sparse_attn.h declares,
and reject bad arguments before any HIP call.  Device pointers here are fake
(aligned, non-null integers) and every call below is built to fail validation,
so nothing is ever launched.
"""
import ctypes
import os
import re

import pytest

import block_sparse_attention_hybrid_amd as sa
import oracle as O

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "sparse_attn.h")
FAKE = ctypes.c_void_p(0x100000)       # aligned, never dereferenced
FAKE_MISALIGNED = ctypes.c_void_p(0x100002)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 12
    lib = sa.lib()
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(sa.EXPORTED)


def geom(**kw):
    base = dict(batch=1, heads=2, frames=4, height=16, width=16, head_dim=64, cube=(4, 4, 4))
    base.update(kw)
    cube = base.pop("cube")
    return sa.make_geom(base["batch"], base["heads"], base["frames"], base["height"],
                        base["width"], base["head_dim"], cube)


@pytest.mark.parametrize("grid,nblk,n_pad", [((4, 16, 16), 16, 1024), ((21, 30, 52), 624, 39936),
                                             ((21, 45, 80), 1440, 92160), ((5, 7, 9), 12, 768)])
def test_geometry_matches_oracle(grid, nblk, n_pad):
    g = geom(frames=grid[0], height=grid[1], width=grid[2])
    got = sa.sparse_attn_geometry(g)
    og = O.Geometry(*grid)
    assert got == (nblk, og.n_real, n_pad) == (og.nblk, og.n_real, og.n_pad)


def test_geometry_other_cube_shapes():
    g = geom(frames=6, height=20, width=20, cube=(2, 4, 8))
    nblk, n_real, n_pad = sa.sparse_attn_geometry(g)
    assert nblk == 3 * 5 * 3 and n_pad == 64 * nblk and n_real == 6 * 20 * 20


def test_ceil_k_matches_worked_example_and_oracle():
    assert sa.sparse_attn_ceil_k(0.03, 1562) == 47
    for k, n in [(0.07, 100), (0.05, 1440), (0.03, 1440), (0.02, 1440), (0.25, 16), (0.0, 16),
                 (1.0, 16), (3.0, 9), (-0.5, 9), (1e-6, 1440), (0.123456, 777)]:
        assert sa.sparse_attn_ceil_k(k, n) == O.ceil_k(k, n), (k, n)
    with pytest.raises(sa.SparseAttnError):
        sa.sparse_attn_ceil_k(float("nan"), 16)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), sa.SA_ERR_UNSUPPORTED),
    (dict(cube=(4, 4, 2)), sa.SA_ERR_INVALID_ARG),
    (dict(cube=(0, 8, 8)), sa.SA_ERR_INVALID_ARG),
    (dict(batch=0), sa.SA_ERR_INVALID_ARG),
    (dict(frames=0), sa.SA_ERR_INVALID_ARG),
    (dict(batch=256, heads=256), sa.SA_ERR_UNSUPPORTED),
])
def test_bad_geometry_rejected(kw, code):
    g = geom(**kw)
    lib = sa.lib()
    assert lib.sparse_attn_reorder(FAKE, ctypes.c_void_p(0x200000), 0, ctypes.byref(g), None) == code
    assert sa.sparse_attn_last_error() != ""
    assert lib.sparse_attn_mask_workspace_bytes(ctypes.byref(g)) == 0


def test_null_and_misaligned_pointers_rejected():
    g = geom()
    lib = sa.lib()
    B = ctypes.byref(g)
    assert lib.sparse_attn_reorder(None, FAKE, 0, B, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_reorder(FAKE, FAKE, 0, B, None) == sa.SA_ERR_INVALID_ARG   # overlap
    assert lib.sparse_attn_reorder(FAKE_MISALIGNED, FAKE, 0, B, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_reorder(FAKE, ctypes.c_void_p(0x200000), 2, B, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_reorder_pool(FAKE, ctypes.c_void_p(0x200000), 0, None, B, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_reorder_pool(FAKE, FAKE, 0, ctypes.c_void_p(0x300000), B, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_reorder_pool(FAKE, ctypes.c_void_p(0x200000), 0, ctypes.c_void_p(0x300004), B,
                                        None) == sa.SA_ERR_INVALID_ARG   # xbar misaligned
    assert lib.sparse_attn_reorder_pool(FAKE, ctypes.c_void_p(0x200000), 3, ctypes.c_void_p(0x300000), B,
                                        None) == sa.SA_ERR_INVALID_ARG   # layout
    P = [ctypes.c_void_p(a) for a in (0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000, 0x700000,
                                      0x800000)]
    assert lib.sparse_attn_reorder_qkv(*P[:7], None, B, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_reorder_qkv(*P[:3], P[0], *P[4:], B, None) == sa.SA_ERR_INVALID_ARG   # qc is q
    assert "input" in sa.sparse_attn_last_error()
    assert lib.sparse_attn_reorder_qkv(*P[:6], ctypes.c_void_p(0x700004), P[7], B, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_unreorder(FAKE, FAKE, FAKE, None, B, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_pool(FAKE, FAKE, None, FAKE, B, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_block_scores(FAKE, FAKE, None, 0.0, B, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_coarse(FAKE, FAKE, None, B, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_router_pool(FAKE, ctypes.c_void_p(0x200000), B, 3, 2, 2, None) == sa.SA_ERR_INVALID_ARG
    assert "tile" in sa.sparse_attn_last_error()
    assert lib.sparse_attn_router_pool(FAKE, ctypes.c_void_p(0x200000), B, 0, 2, 2, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_router_scores(FAKE, FAKE, None, 0.0, B, 2, 2, 2, None, 0,
                                         None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_router_scores(FAKE, FAKE, FAKE, float("inf"), B, 2, 2, 2, None, 0,
                                         None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_router_scores_f32(FAKE, FAKE, None, 0.0, B, 2, 2, 2, None, 0,
                                             None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_router_scores_f32(FAKE, FAKE, ctypes.c_void_p(0x200002), 0.0, B, 2, 2, 2, None, 0,
                                             None) == sa.SA_ERR_INVALID_ARG   # scores misaligned
    assert lib.sparse_attn_router_scores_f32(FAKE, FAKE, FAKE, 0.0, B, 3, 2, 2, None, 0,
                                             None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_coarse(FAKE, ctypes.c_void_p(0x200000), FAKE, B, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 16, B, 0.0, FAKE, None, None, 0,
                               None) == sa.SA_ERR_INVALID_ARG
    assert "lse_c" in sa.sparse_attn_last_error()
    assert lib.sparse_attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 0, B, 0.0, FAKE, FAKE, None, 0,
                               None) == sa.SA_ERR_INVALID_ARG       # cap < 1
    assert lib.sparse_attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 16, B, float("nan"), FAKE, FAKE,
                               None, 0, None) == sa.SA_ERR_INVALID_ARG


def test_select_argument_rules():
    g = geom()                                      # nblk = 16
    lib = sa.lib()
    B = ctypes.byref(g)
    # Top-p may keep every block: cap must cover nblk
    assert lib.sparse_attn_select(FAKE, B, 0.25, 0.5, None, FAKE, FAKE, 15, None) == sa.SA_ERR_CAPACITY
    # Top-k only: cap must cover kc = 4
    assert lib.sparse_attn_select(FAKE, B, 0.25, 0.0, None, FAKE, FAKE, 3, None) == sa.SA_ERR_CAPACITY
    # a row budget replaces Top-k and needs p == 0
    assert lib.sparse_attn_select(FAKE, B, 0.0, 0.5, FAKE, FAKE, FAKE, 16, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_select(FAKE, B, float("inf"), 0.5, None, FAKE, FAKE, 16, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_select(None, B, 0.25, 0.5, None, FAKE, FAKE, 16, None) == sa.SA_ERR_INVALID_ARG
    big = geom(frames=64, height=64, width=68)      # 16*16*17 = 4352 blocks > 4096
    assert lib.sparse_attn_select(FAKE, ctypes.byref(big), 0.1, 0.0, None, FAKE, FAKE, 5000,
                                  None) == sa.SA_ERR_UNSUPPORTED
    # the float32 forms follow the same rules
    assert lib.sparse_attn_select_f32(FAKE, B, 0.25, 0.5, None, FAKE, FAKE, 15, None) == sa.SA_ERR_CAPACITY
    assert lib.sparse_attn_select_f32(FAKE, B, 0.0, 0.5, FAKE, FAKE, FAKE, 16, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_select_f32(None, B, 0.25, 0.5, None, FAKE, FAKE, 16, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_select_f32(ctypes.c_void_p(0x100002), B, 0.25, 0.5, None, FAKE, FAKE, 16,
                                      None) == sa.SA_ERR_INVALID_ARG          # scores misaligned
    assert lib.sparse_attn_select_f32(FAKE, ctypes.byref(big), 0.1, 0.0, None, FAKE, FAKE, 5000,
                                      None) == sa.SA_ERR_UNSUPPORTED
    assert lib.sparse_attn_block_scores_f32(FAKE, FAKE, None, 0.0, B, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_block_scores_f32(FAKE, FAKE, ctypes.c_void_p(0x200002), 0.0, B,
                                            None) == sa.SA_ERR_INVALID_ARG    # scores misaligned
    assert lib.sparse_attn_block_scores_f32(FAKE, FAKE, FAKE, float("nan"), B, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_block_scores_f32(ctypes.c_void_p(0x100008), FAKE, FAKE, 0.0, B,
                                            None) == sa.SA_ERR_INVALID_ARG    # means 8- but not 16-byte aligned
    assert lib.sparse_attn_block_scores_f32(FAKE, ctypes.c_void_p(0x100008), FAKE, 0.0, B,
                                            None) == sa.SA_ERR_INVALID_ARG


def test_build_mask_argument_rules():
    g = geom()
    lib = sa.lib()
    B = ctypes.byref(g)
    need = lib.sparse_attn_mask_workspace_bytes(B)
    assert need >= 3 * 16 * 64 * 8
    assert lib.sparse_attn_build_mask(FAKE, FAKE, B, 128, 0.25, 0.5, None, FAKE, FAKE, 16, FAKE, need,
                                      None) == sa.SA_ERR_UNSUPPORTED
    assert lib.sparse_attn_build_mask(FAKE, FAKE, B, 64, 0.25, 0.5, None, FAKE, FAKE, 16, FAKE, need - 1,
                                      None) == sa.SA_ERR_CAPACITY
    assert lib.sparse_attn_build_mask(FAKE, FAKE, B, 64, 0.25, 0.5, None, FAKE, FAKE, 16,
                                      ctypes.c_void_p(0x100010), need, None) == sa.SA_ERR_INVALID_ARG


def test_python_binding_rejects_non_contiguous():
    import torch
    g = geom()
    x = torch.zeros(1, 2, 1024, 128, dtype=torch.bfloat16)[..., :64]
    with pytest.raises(ValueError):
        sa.sparse_attn_reorder(x, x, 0, g)
    with pytest.raises(TypeError):
        sa.sparse_attn_reorder(torch.zeros(4, dtype=torch.float32), x, 0, g)


def test_grouped_mask_and_fwd_argument_rules():
    g = geom()                                      # nblk = 16, B*H = 2
    lib = sa.lib()
    B = ctypes.byref(g)
    for qg in (0, 3, 8, -2):
        assert lib.sparse_attn_mask_groups_workspace_bytes(B, qg) == 0
        assert lib.sparse_attn_build_mask_groups(FAKE, FAKE, B, qg, 0.25, 0.5, FAKE, FAKE, 16, FAKE, 1 << 20,
                                                 None) == sa.SA_ERR_INVALID_ARG
        assert lib.sparse_attn_fwd_groups(FAKE, FAKE, FAKE, FAKE, FAKE, 16, qg, B, 0.0, FAKE, FAKE,
                                          None) == sa.SA_ERR_INVALID_ARG
    # group means [2, 8, 64] + block means [2, 16, 64] + scores [2, 8, 16], float64, 256-byte regions
    need = lib.sparse_attn_mask_groups_workspace_bytes(B, 2)
    assert need == 2 * 8 * 64 * 8 + 2 * 16 * 64 * 8 + 2 * 8 * 16 * 8
    assert lib.sparse_attn_mask_groups_workspace_bytes(B, 1) == lib.sparse_attn_mask_workspace_bytes(B)
    assert lib.sparse_attn_build_mask_groups(FAKE, FAKE, B, 2, 0.25, 0.5, FAKE, FAKE, 16, FAKE, need - 1,
                                             None) == sa.SA_ERR_CAPACITY
    # Top-p may keep every key block: cap must cover nblk, not nq
    assert lib.sparse_attn_build_mask_groups(FAKE, FAKE, B, 2, 0.25, 0.5, FAKE, FAKE, 15, FAKE, need,
                                             None) == sa.SA_ERR_CAPACITY
    assert lib.sparse_attn_fwd_groups(FAKE, FAKE, None, FAKE, FAKE, 16, 2, B, 0.0, FAKE, FAKE,
                                      None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_fwd_groups(FAKE, FAKE, FAKE, FAKE, FAKE, 16, 2, B, float("nan"), FAKE, FAKE,
                                      None) == sa.SA_ERR_INVALID_ARG


def test_per_sequence_argument_rules():
    g = geom()                                      # nblk = 16
    lib = sa.lib()
    B = ctypes.byref(g)
    need = lib.sparse_attn_sequence_workspace_bytes(B)
    assert need > 0
    assert lib.sparse_attn_select_per_sequence(FAKE, B, 0.25, FAKE, FAKE, 15, FAKE, need,
                                               None) == sa.SA_ERR_CAPACITY       # cap < nblk
    assert lib.sparse_attn_select_per_sequence(FAKE, B, 0.25, FAKE, FAKE, 16, FAKE, need - 1,
                                               None) == sa.SA_ERR_CAPACITY
    assert lib.sparse_attn_select_per_sequence(FAKE, B, float("nan"), FAKE, FAKE, 16, FAKE, need,
                                               None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_select_per_sequence(None, B, 0.25, FAKE, FAKE, 16, FAKE, need,
                                               None) == sa.SA_ERR_INVALID_ARG
    big = geom(frames=64, height=64, width=68)      # 4352 blocks
    assert lib.sparse_attn_select_per_sequence(FAKE, ctypes.byref(big), 0.1, FAKE, FAKE, 5000, FAKE, 1 << 40,
                                               None) == sa.SA_ERR_UNSUPPORTED


def test_ideal_mass_and_recall_argument_rules():
    g = geom()
    lib = sa.lib()
    B = ctypes.byref(g)
    assert lib.sparse_attn_ideal_block_mass(FAKE, FAKE, None, B, 0.0, FAKE, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_ideal_block_mass(FAKE, FAKE, FAKE, B, float("inf"), FAKE, None) == sa.SA_ERR_INVALID_ARG
    need = lib.sparse_attn_recall_workspace_bytes(B)
    assert need >= 2 * 16 * 16 * 4
    assert lib.sparse_attn_mask_recall(FAKE, FAKE, FAKE, 16, B, FAKE, FAKE, need - 1, None) == sa.SA_ERR_CAPACITY
    assert lib.sparse_attn_mask_recall(FAKE, FAKE, FAKE, 0, B, FAKE, FAKE, need, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_mask_recall(FAKE, FAKE, FAKE, 16, B, FAKE_MISALIGNED, FAKE, need,
                                       None) == sa.SA_ERR_INVALID_ARG


def test_whole_path_argument_rules():
    """sparse_attn_attention: every operand buffer is required except the
    row budgets and the slot-major outputs oc / lse_c, which go together."""
    g = geom()
    lib = sa.lib()
    B = ctypes.byref(g)
    F = 0x100000

    def buffers(**kw):
        names = ("q", "k", "v", "qc", "kc", "vc", "qbar", "kbar", "scores", "lut", "counts", "oc", "lse_c",
                 "o", "lse")
        vals = {n: F + 0x10000 * x for x, n in enumerate(names)}     # distinct, aligned, never dereferenced
        vals.update(cap=16, row_budget=None)
        vals.update(kw)
        return sa.PathBuffers(*(vals[n] for n, _ in sa.PathBuffers._fields_))

    def call(buf, k_frac=0.25, p=0.5, chunk=1):
        return lib.sparse_attn_attention(ctypes.byref(buf), B, k_frac, p, 0.0, chunk, None, None)

    assert call(buffers(q=None)) == sa.SA_ERR_INVALID_ARG
    assert call(buffers(o=None)) == sa.SA_ERR_INVALID_ARG
    assert call(buffers(oc=None)) == sa.SA_ERR_INVALID_ARG          # oc without lse_c
    assert "oc and lse_c" in sa.sparse_attn_last_error()
    assert call(buffers(lse_c=None)) == sa.SA_ERR_INVALID_ARG
    assert call(buffers(cap=15)) == sa.SA_ERR_CAPACITY               # Top-p may keep all 16 blocks
    assert call(buffers(), k_frac=float("nan")) == sa.SA_ERR_INVALID_ARG
    assert call(buffers(), chunk=0) == sa.SA_ERR_INVALID_ARG
    # the block means are read in 16-byte pieces
    assert call(buffers(qbar=F + 0x60008)) == sa.SA_ERR_INVALID_ARG
    assert "qbar" in sa.sparse_attn_last_error()
    assert call(buffers(kbar=F + 0x70008)) == sa.SA_ERR_INVALID_ARG
    # the mask phase alone takes no output buffers
    def mask_call(buf, k_frac=0.25, p=0.5):
        return lib.sparse_attn_mask_path(ctypes.byref(buf), B, k_frac, p, None, None)
    assert mask_call(buffers(q=None, o=None, lse=None, oc=None, lse_c=None)) == sa.SA_ERR_INVALID_ARG
    assert "q" in sa.sparse_attn_last_error() and "oc" not in sa.sparse_attn_last_error()
    assert mask_call(buffers(o=None, lse=None, oc=None, cap=15)) == sa.SA_ERR_CAPACITY
    assert mask_call(buffers(scores=None)) == sa.SA_ERR_INVALID_ARG


def test_fused_forward_argument_rules():
    g = geom()
    lib = sa.lib()
    B = ctypes.byref(g)
    O_ = ctypes.c_void_p(0x200000)
    WS = ctypes.c_void_p(0x300000)
    need = sa.sparse_attn_fwd_workspace_bytes(g)
    assert need > 0
    assert lib.sparse_attn_fwd_tokens(FAKE, FAKE, FAKE, FAKE, FAKE, 16, B, 0.0, O_, None, None, 0, None) == \
        sa.SA_ERR_INVALID_ARG
    assert "lse" in sa.sparse_attn_last_error()
    assert lib.sparse_attn_fwd_tokens(FAKE, FAKE, FAKE, FAKE, FAKE, 16, B, 0.0, FAKE_MISALIGNED, FAKE, None, 0,
                                      None) == sa.SA_ERR_INVALID_ARG                 # o misaligned
    assert lib.sparse_attn_fwd_tokens(FAKE, FAKE, FAKE, FAKE, FAKE, 0, B, 0.0, O_, FAKE, None, 0, None) == \
        sa.SA_ERR_INVALID_ARG                                          # cap < 1
    assert lib.sparse_attn_fwd_tokens(FAKE, FAKE, FAKE, FAKE, FAKE, 16, B, float("nan"), O_, FAKE, None, 0,
                                      None) == sa.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_fwd_tokens(FAKE, FAKE, FAKE, FAKE, FAKE, 16, None, 0.0, O_, FAKE, None, 0, None) == \
        sa.SA_ERR_INVALID_ARG                                          # no geometry
    # a schedule workspace below the size the geometry needs, or misaligned
    assert lib.sparse_attn_fwd_tokens(FAKE, FAKE, FAKE, FAKE, FAKE, 16, B, 0.0, O_, FAKE, WS, need - 1, None) == \
        sa.SA_ERR_CAPACITY
    assert lib.sparse_attn_fwd_tokens(FAKE, FAKE, FAKE, FAKE, FAKE, 16, B, 0.0, O_, FAKE, FAKE_MISALIGNED, need,
                                      None) == sa.SA_ERR_INVALID_ARG


def test_forward_workspace_covers_the_row_order():
    """One int32 entry per workgroup of the forward's grid (every row at
    least once), rounded up to 256 bytes."""
    for grid, heads in (((4, 16, 16), 2), ((21, 45, 80), 40), ((1, 1, 1), 1)):
        g = geom(frames=grid[0], height=grid[1], width=grid[2], heads=heads)
        nblk = sa.sparse_attn_geometry(g)[0]
        need = sa.sparse_attn_fwd_workspace_bytes(g)
        assert need % 256 == 0 and need >= 4 * nblk * heads


def test_noalloc_mask_rejects_before_any_launch():
    """The allocation-free mask call validates like sparse_attn_build_mask and
    refuses a (batch, head) whose means and scores exceed its fixed scratch
    array, all before touching the device."""
    lib = sa.lib()
    assert lib.sparse_attn_build_mask_noalloc_scratch_bytes() == 64 << 20
    g = geom(frames=16, height=128, width=128, head_dim=128)           # 4096 blocks: 75.5 MB per head
    assert sa.sparse_attn_geometry(g)[0] == 4096
    rc = lib.sparse_attn_build_mask_noalloc(FAKE, FAKE, ctypes.byref(g), 64, ctypes.c_double(0.03),
                                            ctypes.c_double(0.5), None, FAKE, FAKE, 4096, None)
    assert rc == sa.SA_ERR_CAPACITY
    assert "scratch" in sa.sparse_attn_last_error()
    g2 = geom()
    assert lib.sparse_attn_build_mask_noalloc(FAKE, FAKE, ctypes.byref(g2), 32, ctypes.c_double(0.03),
                                              ctypes.c_double(0.5), None, FAKE, FAKE, 16, None) == sa.SA_ERR_UNSUPPORTED
    assert lib.sparse_attn_build_mask_noalloc(FAKE, FAKE, ctypes.byref(g2), 64, ctypes.c_double(0.03),
                                              ctypes.c_double(0.5), None, FAKE, FAKE, 8, None) == sa.SA_ERR_CAPACITY
    assert lib.sparse_attn_build_mask_noalloc(FAKE_MISALIGNED, FAKE, ctypes.byref(g2), 64, ctypes.c_double(0.03),
                                              ctypes.c_double(0.5), None, FAKE, FAKE, 16, None) == sa.SA_ERR_INVALID_ARG


def test_router_workspace_rules():
    """The one-pass router's scratch, per head: one value per (router row,
    key block) and one running maximum per (router row, column tile of 64
    sub-cubes); for the float32 form also K's three bf16 terms; one 64-bit presence
    word per column tile; three 256-byte alignment pads.  A workspace that
    holds no head is a capacity error and a misaligned one an argument error,
    before any launch."""
    lib = sa.lib()
    for dims, n in (((21, 45, 80), 1440), ((4, 16, 16), 16)):
        for d in (64, 128):
            g = geom(frames=dims[0], height=dims[1], width=dims[2], head_dim=d)
            for sub, G in (((2, 2, 2), 8), ((1, 2, 2), 16), ((4, 4, 4), 1)):
                nt = -(-n * G // 64)
                per_head_elems = nt * nt * 64 * (64 // G) + nt * nt * 64
                for elem in (4, 8):
                    kt = 3 * nt * 64 * d * 2 if elem == 4 else 0
                    want = g.batch * g.heads * (per_head_elems * elem + kt + nt * 8 + 768)
                    assert sa.sparse_attn_router_workspace_bytes(g, sub, elem) == want
    g720 = geom(frames=21, height=45, width=80, head_dim=128)
    # 83.5 MB a head in float32
    assert sa.sparse_attn_router_workspace_bytes(g720, (2, 2, 2), 4) == 2 * (74_649_600 + 8_847_360 + 1_440 + 768)
    assert sa.sparse_attn_router_workspace_bytes(g720, (2, 2, 2), 2) == 0
    assert sa.sparse_attn_router_workspace_bytes(g720, (3, 2, 2), 4) == 0
    one = sa.sparse_attn_router_workspace_bytes(g720, (2, 2, 2), 8) // 2
    assert lib.sparse_attn_router_scores(FAKE, FAKE, FAKE, 0.0, g720, 2, 2, 2, FAKE, one - 1,
                                         None) == sa.SA_ERR_CAPACITY
    assert "workspace" in sa.sparse_attn_last_error()
    assert lib.sparse_attn_router_scores_f32(FAKE, FAKE, FAKE, 0.0, g720, 2, 2, 2, FAKE_MISALIGNED, one,
                                             None) == sa.SA_ERR_INVALID_ARG
