"""MI355X (gfx950) hybrid Top-k U Top-p block-sparse attention for video DiTs.

Thin ctypes binding over ``libsparse_attn.so`` (C ABI in include/sparse_attn.h).
The functions named ``sparse_attn_*`` mirror the C entry points one to one:
they take torch tensors that already live on the GPU, pass their pointers and
the current HIP stream, and raise :class:`SparseAttnError` on a negative status.
Every step of the path runs in the library's HIP kernels; this module only
marshals arguments (and, in the allocating helpers at the bottom, creates
output tensors with ``torch.empty``).  There is no CPU fallback: without the
built library the first call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsparse_attn.so")

SA_OK = 0
SA_ERR_INVALID_ARG = -1
SA_ERR_UNSUPPORTED = -2
SA_ERR_CAPACITY = -3
SA_ERR_HIP = -4
SA_LAYOUT_QK = 0
SA_LAYOUT_V = 1

EXPORTED = (
    "sparse_attn_geometry", "sparse_attn_ceil_k", "sparse_attn_reorder",
    "sparse_attn_reorder_pool", "sparse_attn_reorder_qkv", "sparse_attn_unreorder", "sparse_attn_pool",
    "sparse_attn_block_scores",
    "sparse_attn_select", "sparse_attn_block_scores_f32", "sparse_attn_select_f32",
    "sparse_attn_mask_workspace_bytes", "sparse_attn_fwd_tokens",
    "sparse_attn_build_mask", "sparse_attn_fwd_workspace_bytes", "sparse_attn_fwd",
    "sparse_attn_coarse", "sparse_attn_router_pool", "sparse_attn_router_scores", "sparse_attn_router_scores_f32",
    "sparse_attn_router_workspace_bytes",
    "sparse_attn_bwd_delta", "sparse_attn_transpose_workspace_bytes", "sparse_attn_transpose_lut",
    "sparse_attn_bwd", "sparse_attn_pooled_mass", "sparse_attn_mask_error", "sparse_attn_mask_error_terms",
    "sparse_attn_attention", "sparse_attn_mask_path",
    "sparse_attn_mask_groups_workspace_bytes", "sparse_attn_build_mask_groups", "sparse_attn_fwd_groups",
    "sparse_attn_sequence_workspace_bytes", "sparse_attn_select_per_sequence",
    "sparse_attn_ideal_block_mass", "sparse_attn_recall_workspace_bytes", "sparse_attn_mask_recall",
    "sparse_attn_build_mask_noalloc_scratch_bytes", "sparse_attn_build_mask_noalloc",
    "sparse_attn_last_error",
)


class SparseAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"sparse_attn error {code}: {message}")
        self.code = code


class Geom(ctypes.Structure):
    """sa_geom of the C ABI."""
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "heads", "frames", "height", "width", "head_dim",
        "cube_t", "cube_h", "cube_w")]

    def __repr__(self):
        return ("Geom(batch=%d, heads=%d, grid=%dx%dx%d, head_dim=%d, cube=%dx%dx%d)" %
                (self.batch, self.heads, self.frames, self.height, self.width,
                 self.head_dim, self.cube_t, self.cube_h, self.cube_w))


def make_geom(batch: int, heads: int, frames: int, height: int, width: int,
              head_dim: int, cube: Tuple[int, int, int] = (4, 4, 4)) -> Geom:
    return Geom(batch, heads, frames, height, width, head_dim, *cube)


class BwdArgs(ctypes.Structure):
    """sa_bwd_args of the C ABI."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("q", "k", "v_qk", "k_v", "do_qk", "lse", "delta",
                                               "lut", "counts")] + [("cap", ctypes.c_int32)] + \
               [(n, ctypes.c_void_p) for n in ("lut_t", "counts_t")] + [("cap_t", ctypes.c_int32)]


class PathBuffers(ctypes.Structure):
    """sa_path_buffers of the C ABI."""
    _fields_ = ([(n, ctypes.c_void_p) for n in ("q", "k", "v", "qc", "kc", "vc", "qbar", "kbar", "scores", "lut",
                                                "counts")] + [("cap", ctypes.c_int32)] +
                [(n, ctypes.c_void_p) for n in ("row_budget", "oc", "lse_c", "o", "lse")])


_lib = None
_lock = threading.Lock()
_vp, _i32, _i64, _sz, _f64, _f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                    ctypes.c_size_t, ctypes.c_double, ctypes.c_float)
_GP = ctypes.POINTER(Geom)
_SIGS = {
    "sparse_attn_geometry": (_i32, [_GP, ctypes.POINTER(_i32), ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "sparse_attn_ceil_k": (_i32, [_f64, _i32]),
    "sparse_attn_reorder": (_i32, [_vp, _vp, _i32, _GP, _vp]),
    "sparse_attn_reorder_pool": (_i32, [_vp, _vp, _i32, _vp, _GP, _vp]),
    "sparse_attn_reorder_qkv": (_i32, [_vp] * 8 + [_GP, _vp]),
    "sparse_attn_unreorder": (_i32, [_vp, _vp, _vp, _vp, _GP, _vp]),
    "sparse_attn_pool": (_i32, [_vp, _vp, _vp, _vp, _GP, _vp]),
    "sparse_attn_block_scores": (_i32, [_vp, _vp, _vp, _f64, _GP, _vp]),
    "sparse_attn_block_scores_f32": (_i32, [_vp, _vp, _vp, _f64, _GP, _vp]),
    "sparse_attn_select": (_i32, [_vp, _GP, _f64, _f64, _vp, _vp, _vp, _i32, _vp]),
    "sparse_attn_select_f32": (_i32, [_vp, _GP, _f64, _f64, _vp, _vp, _vp, _i32, _vp]),
    "sparse_attn_mask_workspace_bytes": (_sz, [_GP]),
    "sparse_attn_build_mask": (_i32, [_vp, _vp, _GP, _i32, _f64, _f64, _vp, _vp, _vp, _i32, _vp, _sz, _vp]),
    "sparse_attn_fwd_workspace_bytes": (_sz, [_GP]),
    "sparse_attn_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _GP, _f32, _vp, _vp, _vp, _sz, _vp]),
    "sparse_attn_fwd_tokens": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _GP, _f32, _vp, _vp, _vp, _sz, _vp]),
    "sparse_attn_coarse": (_i32, [_vp, _vp, _vp, _GP, _vp]),
    "sparse_attn_router_pool": (_i32, [_vp, _vp, _GP, _i32, _i32, _i32, _vp]),
    "sparse_attn_router_scores": (_i32, [_vp, _vp, _vp, _f64, _GP, _i32, _i32, _i32, _vp, _sz, _vp]),
    "sparse_attn_router_scores_f32": (_i32, [_vp, _vp, _vp, _f64, _GP, _i32, _i32, _i32, _vp, _sz, _vp]),
    "sparse_attn_router_workspace_bytes": (_sz, [_GP, _i32, _i32, _i32, _i32]),
    "sparse_attn_bwd_delta": (_i32, [_vp, _vp, _vp, _GP, _vp]),
    "sparse_attn_transpose_workspace_bytes": (_sz, [_GP]),
    "sparse_attn_transpose_lut": (_i32, [_vp, _vp, _i32, _vp, _vp, _i32, _GP, _vp, _sz, _vp]),
    "sparse_attn_bwd": (_i32, [ctypes.POINTER(BwdArgs), _GP, _f32, _vp, _vp, _vp, _vp]),
    "sparse_attn_pooled_mass": (_i32, [_vp, _vp, _vp, _i32, _GP, _vp, _vp]),
    "sparse_attn_mask_error": (_i32, [_vp, _vp, _vp, _vp, _GP, _vp, _vp, _vp]),
    "sparse_attn_mask_error_terms": (_i32, [_vp, _vp, _vp, _vp, _GP, _vp, _vp, _vp, _vp, _vp]),
    "sparse_attn_attention": (_i32, [ctypes.POINTER(PathBuffers), _GP, _f64, _f64, _f32, _i32, _vp, _vp]),
    "sparse_attn_mask_path": (_i32, [ctypes.POINTER(PathBuffers), _GP, _f64, _f64, _vp, _vp]),
    "sparse_attn_mask_groups_workspace_bytes": (_sz, [_GP, _i32]),
    "sparse_attn_build_mask_groups": (_i32, [_vp, _vp, _GP, _i32, _f64, _f64, _vp, _vp, _i32, _vp, _sz, _vp]),
    "sparse_attn_fwd_groups": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _GP, _f32, _vp, _vp, _vp]),
    "sparse_attn_sequence_workspace_bytes": (_sz, [_GP]),
    "sparse_attn_select_per_sequence": (_i32, [_vp, _GP, _f64, _vp, _vp, _i32, _vp, _sz, _vp]),
    "sparse_attn_ideal_block_mass": (_i32, [_vp, _vp, _vp, _GP, _f32, _vp, _vp]),
    "sparse_attn_recall_workspace_bytes": (_sz, [_GP]),
    "sparse_attn_mask_recall": (_i32, [_vp, _vp, _vp, _i32, _GP, _vp, _vp, _sz, _vp]),
    "sparse_attn_build_mask_noalloc_scratch_bytes": (_sz, []),
    "sparse_attn_build_mask_noalloc": (_i32, [_vp, _vp, _GP, _i32, _f64, _f64, _vp, _vp, _vp, _i32, _vp]),
    "sparse_attn_last_error": (ctypes.c_char_p, []),
}


def lib() -> ctypes.CDLL:
    """The loaded library, built first when it is missing or older than the
    sources (its recorded source digest no longer matches)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                from . import build as _build
                if not _build.is_current():
                    _build.build()
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in _SIGS.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def _check(code: int) -> int:
    if code < 0:
        msg = lib().sparse_attn_last_error().decode(errors="replace")
        raise SparseAttnError(code, msg)
    return code


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, *tensors):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    for t in tensors:
        if isinstance(t, torch.Tensor) and t.is_cuda:
            return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return None


# ----------------------------------------------------------------------------
# one-to-one C ABI mirrors
# ----------------------------------------------------------------------------
def sparse_attn_geometry(g: Geom) -> Tuple[int, int, int]:
    nblk, n_real, n_pad = _i32(), _i64(), _i64()
    _check(lib().sparse_attn_geometry(ctypes.byref(g), ctypes.byref(nblk), ctypes.byref(n_real),
                                      ctypes.byref(n_pad)))
    return nblk.value, n_real.value, n_pad.value


def sparse_attn_ceil_k(k_frac: float, nblk: int) -> int:
    return _check(lib().sparse_attn_ceil_k(float(k_frac), int(nblk)))


def sparse_attn_reorder(x, xc, layout: int, g: Geom, stream=None) -> None:
    _check(lib().sparse_attn_reorder(_ptr(x, torch.bfloat16, "x"), _ptr(xc, torch.bfloat16, "xc"),
                                     int(layout), ctypes.byref(g), _stream(stream, x)))


def sparse_attn_reorder_pool(x, xc, layout: int, xbar, g: Geom, stream=None) -> None:
    _check(lib().sparse_attn_reorder_pool(_ptr(x, torch.bfloat16, "x"), _ptr(xc, torch.bfloat16, "xc"),
                                          int(layout), _ptr(xbar, torch.float64, "xbar"), ctypes.byref(g),
                                          _stream(stream, x)))


def sparse_attn_reorder_qkv(q, k, v, qc, kc, vc, qbar, kbar, g: Geom, stream=None) -> None:
    _check(lib().sparse_attn_reorder_qkv(_ptr(q, torch.bfloat16, "q"), _ptr(k, torch.bfloat16, "k"),
                                         _ptr(v, torch.bfloat16, "v"), _ptr(qc, torch.bfloat16, "qc"),
                                         _ptr(kc, torch.bfloat16, "kc"), _ptr(vc, torch.bfloat16, "vc"),
                                         _ptr(qbar, torch.float64, "qbar"), _ptr(kbar, torch.float64, "kbar"),
                                         ctypes.byref(g), _stream(stream, q)))


def sparse_attn_unreorder(oc, o, lse_c, lse, g: Geom, stream=None) -> None:
    _check(lib().sparse_attn_unreorder(_ptr(oc, torch.bfloat16, "oc"), _ptr(o, torch.bfloat16, "o"),
                                       _ptr(lse_c, torch.float32, "lse_c"), _ptr(lse, torch.float32, "lse"),
                                       ctypes.byref(g), _stream(stream, oc)))


def sparse_attn_pool(qc, kc, qbar, kbar, g: Geom, stream=None) -> None:
    _check(lib().sparse_attn_pool(_ptr(qc, torch.bfloat16, "qc"), _ptr(kc, torch.bfloat16, "kc"),
                                  _ptr(qbar, torch.float64, "qbar"), _ptr(kbar, torch.float64, "kbar"),
                                  ctypes.byref(g), _stream(stream, qc)))


def sparse_attn_block_scores(qbar, kbar, scores, scale: float, g: Geom, stream=None) -> None:
    _check(lib().sparse_attn_block_scores(_ptr(qbar, torch.float64, "qbar"), _ptr(kbar, torch.float64, "kbar"),
                                          _ptr(scores, torch.float64, "scores"), float(scale),
                                          ctypes.byref(g), _stream(stream, qbar)))


def sparse_attn_select(scores, g: Geom, k_frac: float, p: float, row_budget, lut, counts,
                       cap: int, stream=None) -> None:
    _check(lib().sparse_attn_select(_ptr(scores, torch.float64, "scores"), ctypes.byref(g),
                                    float(k_frac), float(p), _ptr(row_budget, torch.int32, "row_budget"),
                                    _ptr(lut, torch.int32, "lut"), _ptr(counts, torch.int32, "counts"),
                                    int(cap), _stream(stream, scores)))


def sparse_attn_block_scores_f32(qbar, kbar, scores, scale: float, g: Geom, stream=None) -> None:
    _check(lib().sparse_attn_block_scores_f32(_ptr(qbar, torch.float64, "qbar"), _ptr(kbar, torch.float64, "kbar"),
                                              _ptr(scores, torch.float32, "scores"), float(scale),
                                              ctypes.byref(g), _stream(stream, qbar)))


def sparse_attn_select_f32(scores, g: Geom, k_frac: float, p: float, row_budget, lut, counts,
                           cap: int, stream=None) -> None:
    _check(lib().sparse_attn_select_f32(_ptr(scores, torch.float32, "scores"), ctypes.byref(g),
                                        float(k_frac), float(p), _ptr(row_budget, torch.int32, "row_budget"),
                                        _ptr(lut, torch.int32, "lut"), _ptr(counts, torch.int32, "counts"),
                                        int(cap), _stream(stream, scores)))


def sparse_attn_mask_workspace_bytes(g: Geom) -> int:
    return int(lib().sparse_attn_mask_workspace_bytes(ctypes.byref(g)))


def sparse_attn_build_mask(qc, kc, g: Geom, block: int, k_frac: float, p: float, row_budget,
                           lut, counts, cap: int, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sparse_attn_build_mask(_ptr(qc, torch.bfloat16, "qc"), _ptr(kc, torch.bfloat16, "kc"),
                                        ctypes.byref(g), int(block), float(k_frac), float(p),
                                        _ptr(row_budget, torch.int32, "row_budget"),
                                        _ptr(lut, torch.int32, "lut"), _ptr(counts, torch.int32, "counts"),
                                        int(cap), _ptr(workspace, None, "workspace"), ws_bytes,
                                        _stream(stream, qc)))


def sparse_attn_build_mask_noalloc_scratch_bytes() -> int:
    return int(lib().sparse_attn_build_mask_noalloc_scratch_bytes())


def sparse_attn_build_mask_noalloc(qc, kc, g: Geom, block: int, k_frac: float, p: float, row_budget,
                                   lut, counts, cap: int, stream=None) -> None:
    _check(lib().sparse_attn_build_mask_noalloc(_ptr(qc, torch.bfloat16, "qc"), _ptr(kc, torch.bfloat16, "kc"),
                                                ctypes.byref(g), int(block), float(k_frac), float(p),
                                                _ptr(row_budget, torch.int32, "row_budget"),
                                                _ptr(lut, torch.int32, "lut"), _ptr(counts, torch.int32, "counts"),
                                                int(cap), _stream(stream, qc)))


def sparse_attn_fwd_workspace_bytes(g: Geom) -> int:
    return int(lib().sparse_attn_fwd_workspace_bytes(ctypes.byref(g)))


def sparse_attn_fwd_tokens(qc, kc, vc, lut, counts, cap: int, g: Geom, scale: float, o, lse,
                           workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sparse_attn_fwd_tokens(_ptr(qc, torch.bfloat16, "qc"), _ptr(kc, torch.bfloat16, "kc"),
                                        _ptr(vc, torch.bfloat16, "vc"), _ptr(lut, torch.int32, "lut"),
                                        _ptr(counts, torch.int32, "counts"), int(cap), ctypes.byref(g),
                                        float(scale), _ptr(o, torch.bfloat16, "o"),
                                        _ptr(lse, torch.float32, "lse"), _ptr(workspace, None, "workspace"),
                                        ws_bytes, _stream(stream, qc)))


def sparse_attn_fwd(qc, kc, vc, lut, counts, cap: int, g: Geom, scale: float, oc, lse_c,
                    workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sparse_attn_fwd(_ptr(qc, torch.bfloat16, "qc"), _ptr(kc, torch.bfloat16, "kc"),
                                 _ptr(vc, torch.bfloat16, "vc"), _ptr(lut, torch.int32, "lut"),
                                 _ptr(counts, torch.int32, "counts"), int(cap), ctypes.byref(g),
                                 float(scale), _ptr(oc, torch.bfloat16, "oc"),
                                 _ptr(lse_c, torch.float32, "lse_c"), _ptr(workspace, None, "workspace"),
                                 ws_bytes, _stream(stream, qc)))


def sparse_attn_coarse(scores, vbar, oc, g: Geom, stream=None) -> None:
    _check(lib().sparse_attn_coarse(_ptr(scores, torch.float64, "scores"), _ptr(vbar, torch.float64, "vbar"),
                                    _ptr(oc, torch.float64, "oc"), ctypes.byref(g), _stream(stream, scores)))


def sparse_attn_router_pool(xc, xr, g: Geom, sub=(2, 2, 2), stream=None) -> None:
    _check(lib().sparse_attn_router_pool(_ptr(xc, torch.bfloat16, "xc"), _ptr(xr, torch.float64, "xr"),
                                         ctypes.byref(g), int(sub[0]), int(sub[1]), int(sub[2]),
                                         _stream(stream, xc)))


def sparse_attn_router_workspace_bytes(g: Geom, sub=(2, 2, 2), score_bytes: int = 8) -> int:
    return int(lib().sparse_attn_router_workspace_bytes(ctypes.byref(g), int(sub[0]), int(sub[1]), int(sub[2]),
                                                        int(score_bytes)))


def sparse_attn_router_scores(qr, kr, scores, scale: float, g: Geom, sub=(2, 2, 2), workspace=None,
                              stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sparse_attn_router_scores(_ptr(qr, torch.float64, "qr"), _ptr(kr, torch.float64, "kr"),
                                           _ptr(scores, torch.float64, "scores"), float(scale), ctypes.byref(g),
                                           int(sub[0]), int(sub[1]), int(sub[2]),
                                           _ptr(workspace, None, "workspace"), ws_bytes, _stream(stream, qr)))


def sparse_attn_router_scores_f32(qr, kr, scores, scale: float, g: Geom, sub=(2, 2, 2), workspace=None,
                                  stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sparse_attn_router_scores_f32(_ptr(qr, torch.float64, "qr"), _ptr(kr, torch.float64, "kr"),
                                               _ptr(scores, torch.float32, "scores"), float(scale), ctypes.byref(g),
                                               int(sub[0]), int(sub[1]), int(sub[2]),
                                               _ptr(workspace, None, "workspace"), ws_bytes, _stream(stream, qr)))


def sparse_attn_bwd_delta(oc, do_qk, delta, g: Geom, stream=None) -> None:
    _check(lib().sparse_attn_bwd_delta(_ptr(oc, torch.bfloat16, "oc"), _ptr(do_qk, torch.bfloat16, "do_qk"),
                                       _ptr(delta, torch.float32, "delta"), ctypes.byref(g), _stream(stream, oc)))


def sparse_attn_transpose_workspace_bytes(g: Geom) -> int:
    return int(lib().sparse_attn_transpose_workspace_bytes(ctypes.byref(g)))


def sparse_attn_transpose_lut(lut, counts, cap: int, lut_t, counts_t, cap_t: int, g: Geom, workspace,
                              stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sparse_attn_transpose_lut(_ptr(lut, torch.int32, "lut"), _ptr(counts, torch.int32, "counts"),
                                           int(cap), _ptr(lut_t, torch.int32, "lut_t"),
                                           _ptr(counts_t, torch.int32, "counts_t"), int(cap_t), ctypes.byref(g),
                                           _ptr(workspace, None, "workspace"), ws_bytes, _stream(stream, lut)))


def sparse_attn_bwd(args: BwdArgs, g: Geom, scale: float, dq, dk, dv, stream=None, like=None) -> None:
    _check(lib().sparse_attn_bwd(ctypes.byref(args), ctypes.byref(g), float(scale),
                                 _ptr(dq, torch.bfloat16, "dq"), _ptr(dk, torch.bfloat16, "dk"),
                                 _ptr(dv, torch.bfloat16, "dv"), _stream(stream, dq)))


def sparse_attn_pooled_mass(scores, lut, counts, cap: int, g: Geom, mass, stream=None) -> None:
    _check(lib().sparse_attn_pooled_mass(_ptr(scores, torch.float64, "scores"), _ptr(lut, torch.int32, "lut"),
                                         _ptr(counts, torch.int32, "counts"), int(cap), ctypes.byref(g),
                                         _ptr(mass, torch.float64, "mass"), _stream(stream, scores)))


def sparse_attn_mask_error(lse_s, lse_d, oc_s, oc_d, g: Geom, tau, rel_l1, stream=None) -> None:
    _check(lib().sparse_attn_mask_error(_ptr(lse_s, torch.float32, "lse_s"), _ptr(lse_d, torch.float32, "lse_d"),
                                        _ptr(oc_s, torch.bfloat16, "oc_s"), _ptr(oc_d, torch.bfloat16, "oc_d"),
                                        ctypes.byref(g), _ptr(tau, torch.float32, "tau"),
                                        _ptr(rel_l1, torch.float32, "rel_l1"), _stream(stream, lse_s)))


def sparse_attn_mask_error_terms(lse_s, lse_d, oc_s, oc_d, g: Geom, tau, rel_l1, rel_drop, rel_ren,
                                 stream=None) -> None:
    _check(lib().sparse_attn_mask_error_terms(_ptr(lse_s, torch.float32, "lse_s"),
                                              _ptr(lse_d, torch.float32, "lse_d"),
                                              _ptr(oc_s, torch.bfloat16, "oc_s"), _ptr(oc_d, torch.bfloat16, "oc_d"),
                                              ctypes.byref(g), _ptr(tau, torch.float32, "tau"),
                                              _ptr(rel_l1, torch.float32, "rel_l1"),
                                              _ptr(rel_drop, torch.float32, "rel_drop"),
                                              _ptr(rel_ren, torch.float32, "rel_ren"), _stream(stream, lse_s)))


def sparse_attn_attention(buffers: PathBuffers, g: Geom, k_frac: float, p: float, scale: float = 0.0,
                          head_chunk: int = 8, stream=None, aux_stream=None) -> None:
    s = torch.cuda.current_stream().cuda_stream if stream is None else int(stream)
    a = None if aux_stream is None else ctypes.c_void_p(int(aux_stream))
    _check(lib().sparse_attn_attention(ctypes.byref(buffers), ctypes.byref(g), float(k_frac), float(p),
                                       float(scale), int(head_chunk), ctypes.c_void_p(s), a))


def sparse_attn_mask_path(buffers: PathBuffers, g: Geom, k_frac: float, p: float, stream=None,
                          aux_stream=None) -> None:
    s = torch.cuda.current_stream().cuda_stream if stream is None else int(stream)
    a = None if aux_stream is None else ctypes.c_void_p(int(aux_stream))
    _check(lib().sparse_attn_mask_path(ctypes.byref(buffers), ctypes.byref(g), float(k_frac), float(p),
                                       ctypes.c_void_p(s), a))


def sparse_attn_last_error() -> str:
    return lib().sparse_attn_last_error().decode(errors="replace")


# ----------------------------------------------------------------------------
# allocating helpers (torch.empty for outputs, then the entry points above)
# ----------------------------------------------------------------------------
def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def reorder(x: torch.Tensor, g: Geom, layout: int = SA_LAYOUT_QK, stream=None) -> torch.Tensor:
    """Cube-major copy of row-major tokens in the given block layout
    (SA_LAYOUT_QK for queries and keys, SA_LAYOUT_V for values)."""
    nblk, n_real, n_pad = sparse_attn_geometry(g)
    xc = _empty((g.batch, g.heads, n_pad, g.head_dim), torch.bfloat16, x)
    sparse_attn_reorder(x, xc, layout, g, stream)
    return xc


def reorder_pool(x: torch.Tensor, g: Geom, layout: int = SA_LAYOUT_QK, stream=None):
    """Cube-major copy in the given block layout and the float64 block means."""
    nblk, n_real, n_pad = sparse_attn_geometry(g)
    xc = _empty((g.batch, g.heads, n_pad, g.head_dim), torch.bfloat16, x)
    xbar = _empty((g.batch, g.heads, nblk, g.head_dim), torch.float64, x)
    sparse_attn_reorder_pool(x, xc, layout, xbar, g, stream)
    return xc, xbar


def mask_from_pooled(qbar, kbar, g: Geom, k_frac: float, p: float, row_budget=None, cap=None,
                     scores=None, stream=None):
    """Pooled block scores (float32) and hybrid selection from block means:
    the rest of build_mask once reorder_pool has pooled.  Returns (lut, counts)."""
    nblk, _, _ = sparse_attn_geometry(g)
    cap = nblk if cap is None else cap
    if scores is None:
        scores = _empty((g.batch, g.heads, nblk, nblk), torch.float32, qbar)
    lut = _empty((g.batch, g.heads, nblk, cap), torch.int32, qbar)
    counts = _empty((g.batch, g.heads, nblk), torch.int32, qbar)
    sparse_attn_block_scores_f32(qbar, kbar, scores, 0.0, g, stream)
    sparse_attn_select_f32(scores, g, k_frac, p, row_budget, lut, counts, cap, stream)
    return lut, counts


def unreorder(oc: torch.Tensor, lse_c: Optional[torch.Tensor], g: Geom, stream=None):
    nblk, n_real, n_pad = sparse_attn_geometry(g)
    o = _empty((g.batch, g.heads, n_real, g.head_dim), torch.bfloat16, oc)
    lse = None if lse_c is None else _empty((g.batch, g.heads, n_real), torch.float32, oc)
    sparse_attn_unreorder(oc, o, lse_c, lse, g, stream)
    return o, lse


def sparse_attn_mask_groups_workspace_bytes(g: Geom, qgroup: int) -> int:
    return int(lib().sparse_attn_mask_groups_workspace_bytes(ctypes.byref(g), int(qgroup)))


def sparse_attn_build_mask_groups(qc, kc, g: Geom, qgroup: int, k_frac: float, p: float, lut, counts,
                                  cap: int, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sparse_attn_build_mask_groups(_ptr(qc, torch.bfloat16, "qc"), _ptr(kc, torch.bfloat16, "kc"),
                                               ctypes.byref(g), int(qgroup), float(k_frac), float(p),
                                               _ptr(lut, torch.int32, "lut"), _ptr(counts, torch.int32, "counts"),
                                               int(cap), _ptr(workspace, None, "workspace"), ws_bytes,
                                               _stream(stream, qc)))


def sparse_attn_fwd_groups(qc, kc, vc, lut, counts, cap: int, qgroup: int, g: Geom, scale: float, oc, lse_c,
                           stream=None) -> None:
    _check(lib().sparse_attn_fwd_groups(_ptr(qc, torch.bfloat16, "qc"), _ptr(kc, torch.bfloat16, "kc"),
                                        _ptr(vc, torch.bfloat16, "vc"), _ptr(lut, torch.int32, "lut"),
                                        _ptr(counts, torch.int32, "counts"), int(cap), int(qgroup),
                                        ctypes.byref(g), float(scale), _ptr(oc, torch.bfloat16, "oc"),
                                        _ptr(lse_c, torch.float32, "lse_c"), _stream(stream, qc)))


def sparse_attn_sequence_workspace_bytes(g: Geom) -> int:
    return int(lib().sparse_attn_sequence_workspace_bytes(ctypes.byref(g)))


def sparse_attn_select_per_sequence(scores, g: Geom, k_frac: float, lut, counts, cap: int, workspace,
                                    stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sparse_attn_select_per_sequence(_ptr(scores, torch.float64, "scores"), ctypes.byref(g),
                                                 float(k_frac), _ptr(lut, torch.int32, "lut"),
                                                 _ptr(counts, torch.int32, "counts"), int(cap),
                                                 _ptr(workspace, None, "workspace"), ws_bytes,
                                                 _stream(stream, scores)))


def sparse_attn_ideal_block_mass(qc, kc, lse_d, g: Geom, scale: float, mass, stream=None) -> None:
    _check(lib().sparse_attn_ideal_block_mass(_ptr(qc, torch.bfloat16, "qc"), _ptr(kc, torch.bfloat16, "kc"),
                                              _ptr(lse_d, torch.float32, "lse_d"), ctypes.byref(g), float(scale),
                                              _ptr(mass, torch.float64, "mass"), _stream(stream, qc)))


def sparse_attn_recall_workspace_bytes(g: Geom) -> int:
    return int(lib().sparse_attn_recall_workspace_bytes(ctypes.byref(g)))


def sparse_attn_mask_recall(mass, lut, counts, cap: int, g: Geom, recall, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sparse_attn_mask_recall(_ptr(mass, torch.float64, "mass"), _ptr(lut, torch.int32, "lut"),
                                         _ptr(counts, torch.int32, "counts"), int(cap), ctypes.byref(g),
                                         _ptr(recall, torch.float64, "recall"), _ptr(workspace, None, "workspace"),
                                         ws_bytes, _stream(stream, mass)))


def mask_workspace(g: Geom, device) -> torch.Tensor:
    return torch.empty(sparse_attn_mask_workspace_bytes(g), dtype=torch.uint8, device=device)


def build_mask(qc, kc, g: Geom, k_frac: float, p: float, row_budget=None, cap=None,
               workspace=None, stream=None):
    """Kept-block lists (lut [B,H,nblk,cap] int32) and counts [B,H,nblk] int32."""
    nblk, _, _ = sparse_attn_geometry(g)
    cap = nblk if cap is None else cap
    lut = _empty((g.batch, g.heads, nblk, cap), torch.int32, qc)
    counts = _empty((g.batch, g.heads, nblk), torch.int32, qc)
    if workspace is None:
        workspace = mask_workspace(g, qc.device)
    sparse_attn_build_mask(qc, kc, g, 64, k_frac, p, row_budget, lut, counts, cap, workspace, stream)
    return lut, counts


def fwd(qc, kc, vc, lut, counts, g: Geom, scale: float = 0.0, stream=None):
    """Block-sparse forward: cube-major O (bf16) and natural-log LSE (fp32)."""
    _, _, n_pad = sparse_attn_geometry(g)
    oc = _empty((g.batch, g.heads, n_pad, g.head_dim), torch.bfloat16, qc)
    lse_c = _empty((g.batch, g.heads, n_pad), torch.float32, qc)
    nws = sparse_attn_fwd_workspace_bytes(g)
    ws = None if nws == 0 else torch.empty(nws, dtype=torch.uint8, device=qc.device)
    sparse_attn_fwd(qc, kc, vc, lut, counts, lut.shape[-1], g, scale, oc, lse_c, ws, stream)
    return oc, lse_c


def fwd_tokens(qc, kc, vc, lut, counts, g: Geom, scale: float = 0.0, stream=None):
    """Block-sparse forward with the inverse re-indexing fused: O [B,H,N,d]
    (bf16) and natural-log LSE [B,H,N] (fp32) in token order."""
    _, n_real, _ = sparse_attn_geometry(g)
    o = _empty((g.batch, g.heads, n_real, g.head_dim), torch.bfloat16, qc)
    lse = _empty((g.batch, g.heads, n_real), torch.float32, qc)
    ws = torch.empty(sparse_attn_fwd_workspace_bytes(g), dtype=torch.uint8, device=qc.device)
    sparse_attn_fwd_tokens(qc, kc, vc, lut, counts, lut.shape[-1], g, scale, o, lse, ws, stream)
    return o, lse


def build_mask_groups(qc, kc, g: Geom, qgroup: int, k_frac: float, p: float, cap=None, stream=None):
    """Lists of the asymmetric blocks: one per query block of qgroup cubes
    (lut [B,H,nq,cap] int32, counts [B,H,nq] int32, nq = ceil(nblk/qgroup))."""
    nblk, _, _ = sparse_attn_geometry(g)
    nq = -(-nblk // qgroup)
    cap = nblk if cap is None else cap
    lut = _empty((g.batch, g.heads, nq, cap), torch.int32, qc)
    counts = _empty((g.batch, g.heads, nq), torch.int32, qc)
    ws = torch.empty(sparse_attn_mask_groups_workspace_bytes(g, qgroup), dtype=torch.uint8, device=qc.device)
    sparse_attn_build_mask_groups(qc, kc, g, qgroup, k_frac, p, lut, counts, cap, ws, stream)
    return lut, counts


def fwd_groups(qc, kc, vc, lut, counts, g: Geom, qgroup: int, scale: float = 0.0, stream=None):
    """Forward over lists shared by the qgroup cubes of each query block."""
    _, _, n_pad = sparse_attn_geometry(g)
    oc = _empty((g.batch, g.heads, n_pad, g.head_dim), torch.bfloat16, qc)
    lse_c = _empty((g.batch, g.heads, n_pad), torch.float32, qc)
    sparse_attn_fwd_groups(qc, kc, vc, lut, counts, lut.shape[-1], qgroup, g, scale, oc, lse_c, stream)
    return oc, lse_c


def select_per_sequence(scores, g: Geom, k_frac: float, stream=None):
    """Per-sequence Top-K lists of block scores [B,H,nblk,nblk] float64:
    (lut [B,H,nblk,nblk] int32, counts [B,H,nblk] int32)."""
    nblk, _, _ = sparse_attn_geometry(g)
    lut = _empty((g.batch, g.heads, nblk, nblk), torch.int32, scores)
    counts = _empty((g.batch, g.heads, nblk), torch.int32, scores)
    ws = torch.empty(sparse_attn_sequence_workspace_bytes(g), dtype=torch.uint8, device=scores.device)
    sparse_attn_select_per_sequence(scores, g, k_frac, lut, counts, nblk, ws, stream)
    return lut, counts


def attention(q, k, v, g: Geom, k_frac: float, p: float, row_budget=None, stream=None):
    """Whole path on row-major tokens: reorder (pooling Q and K on the way),
    pooled scores and hybrid selection, sparse forward, unreorder.
    Returns (O [B,H,N,d] bf16, LSE [B,H,N] fp32, lut, counts)."""
    qc, qbar = reorder_pool(q, g, SA_LAYOUT_QK, stream)
    kc, kbar = reorder_pool(k, g, SA_LAYOUT_QK, stream)
    vc = reorder(v, g, SA_LAYOUT_V, stream)
    lut, counts = mask_from_pooled(qbar, kbar, g, k_frac, p, row_budget, stream=stream)
    oc, lse_c = fwd(qc, kc, vc, lut, counts, g, stream=stream)
    o, lse = unreorder(oc, lse_c, g, stream)
    return o, lse, lut, counts


def coarse(scores, vbar, g: Geom, stream=None) -> torch.Tensor:
    """Coarse branch output per block: softmax(scores) @ vbar, [B,H,nblk,d] float64."""
    oc = _empty(tuple(vbar.shape), torch.float64, vbar)
    sparse_attn_coarse(scores, vbar, oc, g, stream)
    return oc


def router_mask(qc, kc, g: Geom, k_frac: float, p: float, sub=(2, 2, 2), row_budget=None, cap=None,
                stream=None, dtype=torch.float64, one_pass=True):
    """Hybrid selection on the fine-grained router's block scores, computed in
    `dtype` (torch.float64 or torch.float32), in one pass over the sub-cube
    scores with a scratch workspace (one_pass) or in the two passes that need
    none.  Returns (lut, counts, scores = log P_r)."""
    nblk, _, _ = sparse_attn_geometry(g)
    G = 64 // (sub[0] * sub[1] * sub[2])
    cap = nblk if cap is None else cap
    qr = _empty((g.batch, g.heads, nblk * G, g.head_dim), torch.float64, qc)
    kr = torch.empty_like(qr)
    scores = _empty((g.batch, g.heads, nblk, nblk), dtype, qc)
    lut = _empty((g.batch, g.heads, nblk, cap), torch.int32, qc)
    counts = _empty((g.batch, g.heads, nblk), torch.int32, qc)
    f32 = dtype == torch.float32
    ws = None
    if one_pass:
        ws = torch.empty(sparse_attn_router_workspace_bytes(g, sub, 4 if f32 else 8), dtype=torch.uint8,
                         device=qc.device)
    sparse_attn_router_pool(qc, qr, g, sub, stream)
    sparse_attn_router_pool(kc, kr, g, sub, stream)
    if f32:
        sparse_attn_router_scores_f32(qr, kr, scores, 0.0, g, sub, ws, stream)
        sparse_attn_select_f32(scores, g, k_frac, p, row_budget, lut, counts, cap, stream)
    else:
        sparse_attn_router_scores(qr, kr, scores, 0.0, g, sub, ws, stream)
        sparse_attn_select(scores, g, k_frac, p, row_budget, lut, counts, cap, stream)
    return lut, counts, scores


def transpose_lut(lut, counts, g: Geom, stream=None):
    """For every key block, the ascending list of query blocks that keep it."""
    nblk, _, _ = sparse_attn_geometry(g)
    lut_t = _empty((g.batch, g.heads, nblk, nblk), torch.int32, lut)
    counts_t = _empty((g.batch, g.heads, nblk), torch.int32, lut)
    ws = torch.empty(max(sparse_attn_transpose_workspace_bytes(g), 256), dtype=torch.uint8, device=lut.device)
    sparse_attn_transpose_lut(lut, counts, lut.shape[-1], lut_t, counts_t, nblk, g, ws, stream)
    return lut_t, counts_t


def backward(q, k, v, do, oc, lse_c, lut, counts, g: Geom, scale: float = 0.0, stream=None):
    """Gradients of the block-sparse attention from row-major q, k, v and dO and
    the forward's cube-major O, LSE and lists.  Returns cube-major slot-major
    (dq, dk, dv) bf16; unreorder(x, None, g) brings each to token order."""
    QKL, VL = SA_LAYOUT_QK, SA_LAYOUT_V
    lay = {}
    for name, x, layout in (("q", q, QKL), ("k", k, QKL), ("v_qk", v, QKL), ("k_v", k, VL), ("do_qk", do, QKL)):
        lay[name] = reorder(x, g, layout, stream)
    _, _, n_pad = sparse_attn_geometry(g)
    delta = _empty((g.batch, g.heads, n_pad), torch.float32, q)
    sparse_attn_bwd_delta(oc, lay["do_qk"], delta, g, stream)
    lut_t, counts_t = transpose_lut(lut, counts, g, stream)
    args = BwdArgs(*(lay[n].data_ptr() for n in ("q", "k", "v_qk", "k_v", "do_qk")),
                   lse_c.data_ptr(), delta.data_ptr(), lut.data_ptr(), counts.data_ptr(), lut.shape[-1],
                   lut_t.data_ptr(), counts_t.data_ptr(), lut_t.shape[-1])
    dq, dk, dv = (_empty(tuple(oc.shape), torch.bfloat16, oc) for _ in range(3))
    sparse_attn_bwd(args, g, scale, dq, dk, dv, stream)
    return dq, dk, dv


def mask_quality(qc, kc, vc, lut, counts, scores, g: Geom, stream=None, terms=False):
    """Diagnostics of a kept-block mask: pooled mass per row (from the scores
    the mask was selected on), retained attention mass tau per query and the
    relative L1 error per query block against dense attention (run here with
    every block kept).  Returns (mass, tau, rel_l1), and with terms=True also
    Eq. 8's dropped and renormalisation terms per query block:
    (mass, tau, rel_l1, rel_drop, rel_ren)."""
    nblk, _, n_pad = sparse_attn_geometry(g)
    mass = _empty((g.batch, g.heads, nblk), torch.float64, qc)
    sparse_attn_pooled_mass(scores, lut, counts, lut.shape[-1], g, mass, stream)
    full = _empty((g.batch, g.heads, nblk, nblk), torch.int32, qc)
    full_counts = _empty((g.batch, g.heads, nblk), torch.int32, qc)
    sparse_attn_select(scores, g, 0.0, 1.0, None, full, full_counts, nblk, stream)
    oc_s, lse_s = fwd(qc, kc, vc, lut, counts, g, stream=stream)
    oc_d, lse_d = fwd(qc, kc, vc, full, full_counts, g, stream=stream)
    tau = _empty((g.batch, g.heads, n_pad), torch.float32, qc)
    rel = _empty((g.batch, g.heads, nblk), torch.float32, qc)
    if terms:
        drop, ren = _empty((g.batch, g.heads, nblk), torch.float32, qc), _empty((g.batch, g.heads, nblk), torch.float32, qc)
        sparse_attn_mask_error_terms(lse_s, lse_d, oc_s, oc_d, g, tau, rel, drop, ren, stream)
        return mass, tau, rel, drop, ren
    sparse_attn_mask_error(lse_s, lse_d, oc_s, oc_d, g, tau, rel, stream)
    return mass, tau, rel


def mask_recall(qc, kc, vc, lut, counts, scores, g: Geom, stream=None):
    """Ideal block scores (from a dense run with every block kept) and the
    recall of the lists against them: (mass [B,H,nblk,nblk] float64,
    recall [B,H,nblk] float64).  `scores` are the block scores the lists were
    selected from (used only to list every block for the dense run)."""
    nblk, _, _ = sparse_attn_geometry(g)
    full = _empty((g.batch, g.heads, nblk, nblk), torch.int32, qc)
    full_counts = _empty((g.batch, g.heads, nblk), torch.int32, qc)
    sparse_attn_select(scores, g, 0.0, 1.0, None, full, full_counts, nblk, stream)
    _, lse_d = fwd(qc, kc, vc, full, full_counts, g, stream=stream)
    mass = _empty((g.batch, g.heads, nblk, nblk), torch.float64, qc)
    sparse_attn_ideal_block_mass(qc, kc, lse_d, g, 0.0, mass, stream)
    recall = _empty((g.batch, g.heads, nblk), torch.float64, qc)
    ws = torch.empty(sparse_attn_recall_workspace_bytes(g), dtype=torch.uint8, device=qc.device)
    sparse_attn_mask_recall(mass, lut, counts, lut.shape[-1], g, recall, ws, stream)
    return mass, recall


def path_buffers(q, k, v, g: Geom, row_budget=None, slot_major: bool = True):
    """Allocate every buffer of sparse_attn_attention for row-major q, k, v.
    slot_major=False leaves oc and lse_c NULL (the forward then writes token
    order directly).  Returns (PathBuffers, dict of the tensors, which must
    outlive the call)."""
    nblk, n_real, n_pad = sparse_attn_geometry(g)
    B, H, d = g.batch, g.heads, g.head_dim
    t = dict(q=q, k=k, v=v)
    for n in ("qc", "kc", "vc") + (("oc",) if slot_major else ()):
        t[n] = _empty((B, H, n_pad, d), torch.bfloat16, q)
    t["qbar"], t["kbar"] = (_empty((B, H, nblk, d), torch.float64, q) for _ in range(2))
    t["scores"] = _empty((B, H, nblk, nblk), torch.float64, q)
    t["lut"] = _empty((B, H, nblk, nblk), torch.int32, q)
    t["counts"] = _empty((B, H, nblk), torch.int32, q)
    t["lse_c"] = _empty((B, H, n_pad), torch.float32, q) if slot_major else None
    t["o"] = _empty((B, H, n_real, d), torch.bfloat16, q)
    t["lse"] = _empty((B, H, n_real), torch.float32, q)
    for n in ("q", "k", "v"):
        _ptr(t[n], torch.bfloat16, n)
    ptr = lambda n: None if t.get(n) is None else t[n].data_ptr()
    buf = PathBuffers(ptr("q"), ptr("k"), ptr("v"), ptr("qc"), ptr("kc"), ptr("vc"), ptr("qbar"), ptr("kbar"),
                      ptr("scores"), ptr("lut"), ptr("counts"), nblk,
                      None if row_budget is None else row_budget.data_ptr(),
                      ptr("oc"), ptr("lse_c"), ptr("o"), ptr("lse"))
    t["row_budget"] = row_budget
    return buf, t


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
