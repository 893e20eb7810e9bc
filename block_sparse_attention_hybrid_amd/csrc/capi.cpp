// C ABI of the sparse-attention library: argument validation on the host, then
// asynchronous kernel launches on the caller's stream.  Every check runs
// before any HIP call, so an invalid call touches no device state.
#include "../../include/sparse_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "sa_launch.h"

namespace {

thread_local char g_last_error[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int32_t ok() {
  g_last_error[0] = '\0';
  return SA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kMaxSelectBlocks = 4096;
constexpr size_t kWsAlign = 256;

size_t round_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Validates the geometry and fills the device-side description.
int32_t make_geom(const sa_geom* g, sa::Geom& d) {
  if (g == nullptr) return fail(SA_ERR_INVALID_ARG, "geometry pointer is NULL");
  if (g->batch < 1 || g->heads < 1) return fail(SA_ERR_INVALID_ARG, "batch and heads must be >= 1");
  if (g->frames < 1 || g->height < 1 || g->width < 1)
    return fail(SA_ERR_INVALID_ARG, "frames, height and width must be >= 1");
  if (g->cube_t < 1 || g->cube_h < 1 || g->cube_w < 1 ||
      (long long)g->cube_t * g->cube_h * g->cube_w != 64)
    return fail(SA_ERR_INVALID_ARG, "cube_t*cube_h*cube_w must be 64 (got %d x %d x %d)", g->cube_t,
                g->cube_h, g->cube_w);
  if (g->head_dim != 64 && g->head_dim != 128)
    return fail(SA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", g->head_dim);
  if ((long long)g->batch * g->heads > 65535)
    return fail(SA_ERR_UNSUPPORTED, "batch*heads must be <= 65535 (got %lld)", (long long)g->batch * g->heads);
  d.batch = g->batch;
  d.heads = g->heads;
  d.frames = g->frames;
  d.height = g->height;
  d.width = g->width;
  d.d = g->head_dim;
  d.ct = g->cube_t;
  d.ch = g->cube_h;
  d.cw = g->cube_w;
  const long long nt = (g->frames + g->cube_t - 1) / g->cube_t;
  const long long nh = (g->height + g->cube_h - 1) / g->cube_h;
  const long long nw = (g->width + g->cube_w - 1) / g->cube_w;
  const long long nblk = nt * nh * nw;
  if (nblk > (1 << 24)) return fail(SA_ERR_UNSUPPORTED, "too many blocks per head (%lld)", nblk);
  const long long rows = nblk * g->batch * g->heads;
  if (rows > 0x7fffffffLL) return fail(SA_ERR_UNSUPPORTED, "batch*heads*blocks exceeds 2^31");
  d.nt = (int)nt;
  d.nh = (int)nh;
  d.nw = (int)nw;
  d.nblk = (int)nblk;
  d.n_real = (long long)g->frames * g->height * g->width;
  d.n_pad = nblk * 64;
  return SA_OK;
}

int32_t check_ptr(const void* p, size_t align, const char* name) {
  if (p == nullptr) return fail(SA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, align)) return fail(SA_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
  return SA_OK;
}

int32_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define SA_TRY(expr)          \
  do {                        \
    const int32_t rc_ = (expr); \
    if (rc_ != SA_OK) return rc_; \
  } while (0)

int32_t ceil_k_impl(double k_frac, int32_t nblk) {
  if (nblk < 0 || !std::isfinite(k_frac)) return SA_ERR_INVALID_ARG;
  if (nblk == 0) return 0;
  const double c = std::ceil(k_frac * (double)nblk - 1e-9);
  if (c <= 0.0) return 0;
  if (c >= (double)nblk) return nblk;
  return (int32_t)c;
}

int32_t check_select_args(const sa::Geom& d, double k_frac, double p, const int32_t* row_budget,
                          const int32_t* lut, const int32_t* counts, int32_t cap, int& kc) {
  if (d.nblk > kMaxSelectBlocks)
    return fail(SA_ERR_UNSUPPORTED, "selection supports at most %d blocks per head (got %d)",
                kMaxSelectBlocks, d.nblk);
  if (!std::isfinite(k_frac) || !std::isfinite(p)) return fail(SA_ERR_INVALID_ARG, "k_frac and p must be finite");
  if (row_budget != nullptr && p != 0.0)
    return fail(SA_ERR_INVALID_ARG, "a row budget replaces Top-k and requires p == 0");
  if (row_budget != nullptr) SA_TRY(check_ptr(row_budget, 4, "row_budget"));
  SA_TRY(check_ptr(lut, 4, "lut"));
  SA_TRY(check_ptr(counts, 4, "counts"));
  kc = ceil_k_impl(k_frac, d.nblk);
  const int need = (p > 0.0 || row_budget != nullptr) ? d.nblk : kc;
  if (cap < 1 || cap < need)
    return fail(SA_ERR_CAPACITY, "cap %d is below the largest possible row count %d", cap, need);
  return SA_OK;
}

size_t mask_ws_bytes(const sa::Geom& d) {
  const size_t rows = (size_t)d.batch * d.heads * d.nblk;
  return 2 * round_up(rows * d.d * sizeof(double)) + round_up(rows * d.nblk * sizeof(double));
}

// qgroup in {1, 2, 4}; returns log2(qgroup) in shift
int32_t check_qgroup(int32_t qgroup, int& shift) {
  if (qgroup != 1 && qgroup != 2 && qgroup != 4)
    return fail(SA_ERR_INVALID_ARG, "qgroup must be 1, 2 or 4 (got %d)", qgroup);
  shift = qgroup == 1 ? 0 : (qgroup == 2 ? 1 : 2);
  return SA_OK;
}

// group means of Q [rows_q, d], block means of K [rows, d], scores [rows_q, nblk]
size_t mask_groups_ws_bytes(const sa::Geom& d, int qgroup) {
  const size_t bh = (size_t)d.batch * d.heads;
  const size_t nq = (size_t)(d.nblk + qgroup - 1) / qgroup;
  return round_up(bh * nq * d.d * sizeof(double)) + round_up(bh * d.nblk * d.d * sizeof(double)) +
         round_up(bh * nq * d.nblk * sizeof(double));
}

}  // namespace

int32_t sa_validate_build_mask(const void* qc, const void* kc, const sa_geom* g, int32_t block, double k_frac,
                               double p, const int32_t* row_budget, const int32_t* lut, const int32_t* counts,
                               int32_t cap, sa::Geom& d, int& kcount);

extern "C" {

int32_t sparse_attn_geometry(const sa_geom* g, int32_t* nblk, int64_t* n_real, int64_t* n_pad) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  if (nblk) *nblk = d.nblk;
  if (n_real) *n_real = d.n_real;
  if (n_pad) *n_pad = d.n_pad;
  return ok();
}

int32_t sparse_attn_ceil_k(double k_frac, int32_t nblk) {
  const int32_t r = ceil_k_impl(k_frac, nblk);
  if (r < 0) return fail(r, "ceil_k needs nblk >= 0 and a finite k_frac");
  return r;
}

int32_t sparse_attn_reorder(const void* x, void* xc, int32_t layout, const sa_geom* g, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(x, 16, "x"));
  SA_TRY(check_ptr(xc, 16, "xc"));
  if (layout != SA_LAYOUT_QK && layout != SA_LAYOUT_V)
    return fail(SA_ERR_INVALID_ARG, "layout must be SA_LAYOUT_QK or SA_LAYOUT_V (got %d)", layout);
  if (x == xc) return fail(SA_ERR_INVALID_ARG, "x and xc must not overlap");
  return hip_status(sa::launch_reorder(x, xc, layout, d, (hipStream_t)stream), "reorder launch");
}

int32_t sparse_attn_reorder_pool(const void* x, void* xc, int32_t layout, double* xbar, const sa_geom* g,
                                 void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(x, 16, "x"));
  SA_TRY(check_ptr(xc, 16, "xc"));
  SA_TRY(check_ptr(xbar, 8, "xbar"));
  if (layout != SA_LAYOUT_QK && layout != SA_LAYOUT_V)
    return fail(SA_ERR_INVALID_ARG, "layout must be SA_LAYOUT_QK or SA_LAYOUT_V (got %d)", layout);
  if (x == xc) return fail(SA_ERR_INVALID_ARG, "x and xc must not overlap");
  return hip_status(sa::launch_reorder_pool(x, xc, layout, xbar, d, (hipStream_t)stream), "reorder_pool launch");
}

int32_t sparse_attn_reorder_qkv(const void* q, const void* k, const void* v, void* qc, void* kc, void* vc,
                                double* qbar, double* kbar, const sa_geom* g, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(q, 16, "q"));
  SA_TRY(check_ptr(k, 16, "k"));
  SA_TRY(check_ptr(v, 16, "v"));
  SA_TRY(check_ptr(qc, 16, "qc"));
  SA_TRY(check_ptr(kc, 16, "kc"));
  SA_TRY(check_ptr(vc, 16, "vc"));
  SA_TRY(check_ptr(qbar, 8, "qbar"));
  SA_TRY(check_ptr(kbar, 8, "kbar"));
  const void* in[3] = {q, k, v};
  const void* out[5] = {qc, kc, vc, qbar, kbar};
  for (const void* a : in)
    for (const void* b : out)
      if (a == b) return fail(SA_ERR_INVALID_ARG, "an output of reorder_qkv is also one of its inputs");
  return hip_status(sa::launch_reorder_qkv(q, k, v, qc, kc, vc, qbar, kbar, d, (hipStream_t)stream),
                    "reorder_qkv launch");
}

int32_t sparse_attn_unreorder(const void* oc, void* o, const float* lse_c, float* lse,
                              const sa_geom* g, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(oc, 16, "oc"));
  SA_TRY(check_ptr(o, 16, "o"));
  if ((lse_c == nullptr) != (lse == nullptr))
    return fail(SA_ERR_INVALID_ARG, "lse_c and lse must both be given or both be NULL");
  if (lse_c != nullptr) {
    SA_TRY(check_ptr(lse_c, 4, "lse_c"));
    SA_TRY(check_ptr(lse, 4, "lse"));
  }
  return hip_status(sa::launch_unreorder(oc, o, lse_c, lse, d, (hipStream_t)stream), "unreorder launch");
}

int32_t sparse_attn_pool(const void* qc, const void* kc, double* qbar, double* kbar, const sa_geom* g,
                         void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(qc, 16, "qc"));
  SA_TRY(check_ptr(kc, 16, "kc"));
  SA_TRY(check_ptr(qbar, 8, "qbar"));
  SA_TRY(check_ptr(kbar, 8, "kbar"));
  return hip_status(sa::launch_pool(qc, kc, qbar, kbar, d, (hipStream_t)stream), "pool launch");
}

int32_t sparse_attn_coarse(const double* scores, const double* vbar, double* oc, const sa_geom* g, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(scores, 8, "scores"));
  SA_TRY(check_ptr(vbar, 8, "vbar"));
  SA_TRY(check_ptr(oc, 8, "oc"));
  if ((const void*)oc == (const void*)scores || (const void*)oc == (const void*)vbar)
    return fail(SA_ERR_INVALID_ARG, "oc must not overlap its inputs");
  return hip_status(sa::launch_coarse(scores, vbar, oc, d, (hipStream_t)stream), "coarse launch");
}

static int32_t check_subcube(const sa::Geom& d, int32_t rt, int32_t rh, int32_t rw) {
  if (rt < 1 || rh < 1 || rw < 1 || d.ct % rt || d.ch % rh || d.cw % rw)
    return fail(SA_ERR_INVALID_ARG, "sub-cube %d x %d x %d must tile the %d x %d x %d cube", rt, rh, rw, d.ct,
                d.ch, d.cw);
  const long long G = 64 / ((long long)rt * rh * rw);
  if ((long long)d.nblk * G * d.batch * d.heads > 0x7fffffffLL)
    return fail(SA_ERR_UNSUPPORTED, "too many sub-cubes (%lld per head)", (long long)d.nblk * G);
  return SA_OK;
}

int32_t sparse_attn_router_pool(const void* xc, double* xr, const sa_geom* g, int32_t rt, int32_t rh, int32_t rw,
                                void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_subcube(d, rt, rh, rw));
  SA_TRY(check_ptr(xc, 16, "xc"));
  SA_TRY(check_ptr(xr, 8, "xr"));
  return hip_status(sa::launch_router_pool(xc, xr, d, rt, rh, rw, (hipStream_t)stream), "router_pool launch");
}

size_t sparse_attn_router_workspace_bytes(const sa_geom* g, int32_t rt, int32_t rh, int32_t rw,
                                          int32_t score_bytes) {
  sa::Geom d;
  if (make_geom(g, d) != SA_OK || check_subcube(d, rt, rh, rw) != SA_OK) return 0;
  if (score_bytes != 4 && score_bytes != 8) return 0;
  return sa::router_workspace_bytes(d, rt, rh, rw, (size_t)score_bytes, d.batch * d.heads);
}

namespace {

// Arguments shared by the two router entry points; the workspace, when given,
// must hold at least one (batch*head)'s share of the one-pass scratch.
int32_t check_router(const double* qr, const double* kr, const void* scores, size_t score_bytes, double& scale,
                     const sa_geom* g, int32_t rt, int32_t rh, int32_t rw, void* workspace,
                     size_t workspace_bytes, sa::Geom& d) {
  SA_TRY(make_geom(g, d));
  SA_TRY(check_subcube(d, rt, rh, rw));
  SA_TRY(check_ptr(qr, 8, "qr"));
  SA_TRY(check_ptr(kr, 8, "kr"));
  SA_TRY(check_ptr(scores, score_bytes, "scores"));
  if (!std::isfinite(scale)) return fail(SA_ERR_INVALID_ARG, "scale must be finite");
  if (scale <= 0.0) scale = 1.0 / std::sqrt((double)d.d);
  if (workspace != nullptr) {
    SA_TRY(check_ptr(workspace, 256, "workspace"));
    const size_t one = sa::router_workspace_bytes(d, rt, rh, rw, score_bytes, 1);
    if (workspace_bytes < one)
      return fail(SA_ERR_CAPACITY, "router workspace of %zu bytes holds no head (%zu needed per head)",
                  workspace_bytes, one);
  }
  return SA_OK;
}

}  // namespace

int32_t sparse_attn_router_scores(const double* qr, const double* kr, double* scores, double scale,
                                  const sa_geom* g, int32_t rt, int32_t rh, int32_t rw, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  sa::Geom d;
  SA_TRY(check_router(qr, kr, scores, 8, scale, g, rt, rh, rw, workspace, workspace_bytes, d));
  return hip_status(sa::launch_router(qr, kr, scores, scale, d, rt, rh, rw, (hipStream_t)stream, workspace,
                                      workspace_bytes),
                    "router launch");
}

int32_t sparse_attn_router_scores_f32(const double* qr, const double* kr, float* scores, double scale,
                                      const sa_geom* g, int32_t rt, int32_t rh, int32_t rw, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  sa::Geom d;
  SA_TRY(check_router(qr, kr, scores, 4, scale, g, rt, rh, rw, workspace, workspace_bytes, d));
  return hip_status(sa::launch_router(qr, kr, scores, scale, d, rt, rh, rw, (hipStream_t)stream, workspace,
                                      workspace_bytes),
                    "router launch");
}

int32_t sparse_attn_bwd_delta(const void* oc, const void* do_qk, float* delta, const sa_geom* g, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(oc, 16, "oc"));
  SA_TRY(check_ptr(do_qk, 16, "do_qk"));
  SA_TRY(check_ptr(delta, 4, "delta"));
  return hip_status(sa::launch_bwd_delta(oc, do_qk, delta, d, (hipStream_t)stream), "bwd_delta launch");
}

size_t sparse_attn_transpose_workspace_bytes(const sa_geom* g) {
  sa::Geom d;
  if (make_geom(g, d) != SA_OK) return 0;
  return sa::transpose_workspace_bytes(d);
}

int32_t sparse_attn_transpose_lut(const int32_t* lut, const int32_t* counts, int32_t cap, int32_t* lut_t,
                                  int32_t* counts_t, int32_t cap_t, const sa_geom* g, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(lut, 4, "lut"));
  SA_TRY(check_ptr(counts, 4, "counts"));
  SA_TRY(check_ptr(lut_t, 4, "lut_t"));
  SA_TRY(check_ptr(counts_t, 4, "counts_t"));
  SA_TRY(check_ptr(workspace, 256, "workspace"));
  if (cap < 1) return fail(SA_ERR_INVALID_ARG, "cap must be >= 1");
  if (cap_t < d.nblk) return fail(SA_ERR_CAPACITY, "cap_t %d is below nblk %d", cap_t, d.nblk);
  if (workspace_bytes < sa::transpose_workspace_bytes(d))
    return fail(SA_ERR_CAPACITY, "workspace of %zu bytes is below the %zu needed", workspace_bytes,
                sa::transpose_workspace_bytes(d));
  return hip_status(sa::launch_transpose_lut(lut, counts, cap, lut_t, counts_t, cap_t, d, workspace,
                                             (hipStream_t)stream),
                    "transpose_lut launch");
}

int32_t sparse_attn_bwd(const sa_bwd_args* a, const sa_geom* g, float scale, void* dq, void* dk, void* dv,
                        void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  if (a == nullptr) return fail(SA_ERR_INVALID_ARG, "args pointer is NULL");
  SA_TRY(check_ptr(a->q, 16, "q"));
  SA_TRY(check_ptr(a->k, 16, "k"));
  SA_TRY(check_ptr(a->v_qk, 16, "v_qk"));
  SA_TRY(check_ptr(a->k_v, 16, "k_v"));
  SA_TRY(check_ptr(a->do_qk, 16, "do_qk"));
  SA_TRY(check_ptr(a->lse, 16, "lse"));
  SA_TRY(check_ptr(a->delta, 16, "delta"));
  SA_TRY(check_ptr(a->lut, 4, "lut"));
  SA_TRY(check_ptr(a->counts, 4, "counts"));
  SA_TRY(check_ptr(a->lut_t, 4, "lut_t"));
  SA_TRY(check_ptr(a->counts_t, 4, "counts_t"));
  SA_TRY(check_ptr(dq, 16, "dq"));
  SA_TRY(check_ptr(dk, 16, "dk"));
  SA_TRY(check_ptr(dv, 16, "dv"));
  if (a->cap < 1 || a->cap_t < 1) return fail(SA_ERR_INVALID_ARG, "cap and cap_t must be >= 1");
  if (dq == dk || dq == dv || dk == dv) return fail(SA_ERR_INVALID_ARG, "dq, dk and dv must not overlap");
  if (!std::isfinite(scale)) return fail(SA_ERR_INVALID_ARG, "scale must be finite");
  if (scale <= 0.f) scale = 1.f / std::sqrt((float)d.d);
  sa::BwdArgs b;
  b.q = a->q;
  b.k = a->k;
  b.v_qk = a->v_qk;
  b.k_v = a->k_v;
  b.do_qk = a->do_qk;
  b.lse = a->lse;
  b.delta = a->delta;
  b.lut = a->lut;
  b.counts = a->counts;
  b.cap = a->cap;
  b.lut_t = a->lut_t;
  b.counts_t = a->counts_t;
  b.cap_t = a->cap_t;
  return hip_status(sa::launch_bwd(b, d, scale, dq, dk, dv, (hipStream_t)stream), "bwd launch");
}

int32_t sparse_attn_pooled_mass(const double* scores, const int32_t* lut, const int32_t* counts, int32_t cap,
                                const sa_geom* g, double* mass, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(scores, 8, "scores"));
  SA_TRY(check_ptr(lut, 4, "lut"));
  SA_TRY(check_ptr(counts, 4, "counts"));
  SA_TRY(check_ptr(mass, 8, "mass"));
  if (cap < 1) return fail(SA_ERR_INVALID_ARG, "cap must be >= 1");
  return hip_status(sa::launch_pooled_mass(scores, lut, counts, cap, d, mass, (hipStream_t)stream),
                    "pooled_mass launch");
}

int32_t sparse_attn_mask_error(const float* lse_s, const float* lse_d, const void* oc_s, const void* oc_d,
                               const sa_geom* g, float* tau, float* rel_l1, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(lse_s, 4, "lse_s"));
  SA_TRY(check_ptr(lse_d, 4, "lse_d"));
  SA_TRY(check_ptr(oc_s, 16, "oc_s"));
  SA_TRY(check_ptr(oc_d, 16, "oc_d"));
  SA_TRY(check_ptr(tau, 4, "tau"));
  SA_TRY(check_ptr(rel_l1, 4, "rel_l1"));
  return hip_status(sa::launch_mask_error(lse_s, lse_d, oc_s, oc_d, d, tau, rel_l1, (hipStream_t)stream),
                    "mask_error launch");
}

int32_t sparse_attn_mask_error_terms(const float* lse_s, const float* lse_d, const void* oc_s, const void* oc_d,
                                     const sa_geom* g, float* tau, float* rel_l1, float* rel_drop,
                                     float* rel_ren, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(lse_s, 4, "lse_s"));
  SA_TRY(check_ptr(lse_d, 4, "lse_d"));
  SA_TRY(check_ptr(oc_s, 16, "oc_s"));
  SA_TRY(check_ptr(oc_d, 16, "oc_d"));
  SA_TRY(check_ptr(tau, 4, "tau"));
  SA_TRY(check_ptr(rel_l1, 4, "rel_l1"));
  SA_TRY(check_ptr(rel_drop, 4, "rel_drop"));
  SA_TRY(check_ptr(rel_ren, 4, "rel_ren"));
  return hip_status(sa::launch_mask_error(lse_s, lse_d, oc_s, oc_d, d, tau, rel_l1, (hipStream_t)stream,
                                          rel_drop, rel_ren),
                    "mask_error launch");
}

}  // extern "C"

int32_t sa_hip_status(hipError_t e, const char* what) { return hip_status(e, what); }

int32_t sa_fail(int32_t code, const char* msg) { return fail(code, "%s", msg); }

// Arguments of sparse_attn_build_mask other than the workspace (shared with
// the allocation-free form).
int32_t sa_validate_build_mask(const void* qc, const void* kc, const sa_geom* g, int32_t block, double k_frac,
                               double p, const int32_t* row_budget, const int32_t* lut, const int32_t* counts,
                               int32_t cap, sa::Geom& d, int& kcount) {
  SA_TRY(make_geom(g, d));
  if (block != 64) return fail(SA_ERR_UNSUPPORTED, "block must be 64 (got %d)", block);
  SA_TRY(check_ptr(qc, 16, "qc"));
  SA_TRY(check_ptr(kc, 16, "kc"));
  SA_TRY(check_select_args(d, k_frac, p, row_budget, lut, counts, cap, kcount));
  return ok();
}

// outputs = false: the mask phase only (oc, lse_c, o and lse are not used)
int32_t sa_validate_path(const sa_path_buffers* b, const sa_geom* g, double k_frac, double p, float scale,
                         int32_t head_chunk, bool outputs, sa::Geom& d, int& kcount, float& scale_out) {
  SA_TRY(make_geom(g, d));
  if (b == nullptr) return fail(SA_ERR_INVALID_ARG, "buffers pointer is NULL");
  if (d.nblk > 64 * 65535) return fail(SA_ERR_UNSUPPORTED, "too many blocks for the score grid");
  SA_TRY(check_ptr(b->q, 16, "q"));
  SA_TRY(check_ptr(b->k, 16, "k"));
  SA_TRY(check_ptr(b->v, 16, "v"));
  SA_TRY(check_ptr(b->qc, 16, "qc"));
  SA_TRY(check_ptr(b->kc, 16, "kc"));
  SA_TRY(check_ptr(b->vc, 16, "vc"));
  SA_TRY(check_ptr(b->qbar, 16, "qbar"));   // read in 16-byte pieces by the float32 block scores
  SA_TRY(check_ptr(b->kbar, 16, "kbar"));
  SA_TRY(check_ptr(b->scores, 8, "scores"));
  // oc and lse_c: both given (slot-major O and LSE are written too) or both NULL
  if (outputs) {
    if ((b->oc == nullptr) != (b->lse_c == nullptr))
      return fail(SA_ERR_INVALID_ARG, "oc and lse_c must both be given or both be NULL");
    if (b->oc != nullptr) {
      SA_TRY(check_ptr(b->oc, 16, "oc"));
      SA_TRY(check_ptr(b->lse_c, 4, "lse_c"));
    }
    SA_TRY(check_ptr(b->o, 16, "o"));
    SA_TRY(check_ptr(b->lse, 4, "lse"));
  }
  if (b->q == b->qc || b->k == b->kc || b->v == b->vc) return fail(SA_ERR_INVALID_ARG, "inputs and outputs overlap");
  SA_TRY(check_select_args(d, k_frac, p, b->row_budget, b->lut, b->counts, b->cap, kcount));
  if (head_chunk < 1) return fail(SA_ERR_INVALID_ARG, "head_chunk must be >= 1");
  if (!std::isfinite(scale)) return fail(SA_ERR_INVALID_ARG, "scale must be finite");
  scale_out = scale <= 0.f ? 1.f / std::sqrt((float)d.d) : scale;
  return ok();
}

extern "C" {

int32_t sparse_attn_block_scores(const double* qbar, const double* kbar, double* scores, double scale,
                                 const sa_geom* g, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  if (d.nblk > 64 * 65535) return fail(SA_ERR_UNSUPPORTED, "too many blocks for the score grid");
  SA_TRY(check_ptr(qbar, 8, "qbar"));
  SA_TRY(check_ptr(kbar, 8, "kbar"));
  SA_TRY(check_ptr(scores, 8, "scores"));
  if (!std::isfinite(scale)) return fail(SA_ERR_INVALID_ARG, "scale must be finite");
  if (scale <= 0.0) scale = 1.0 / std::sqrt((double)d.d);
  return hip_status(sa::launch_block_scores(qbar, kbar, scores, scale, d, (hipStream_t)stream),
                    "block score launch");
}

int32_t sparse_attn_block_scores_f32(const double* qbar, const double* kbar, float* scores, double scale,
                                     const sa_geom* g, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  if (d.nblk > 64 * 65535) return fail(SA_ERR_UNSUPPORTED, "too many blocks for the score grid");
  SA_TRY(check_ptr(qbar, 16, "qbar"));
  SA_TRY(check_ptr(kbar, 16, "kbar"));
  SA_TRY(check_ptr(scores, 4, "scores"));
  if (!std::isfinite(scale)) return fail(SA_ERR_INVALID_ARG, "scale must be finite");
  if (scale <= 0.0) scale = 1.0 / std::sqrt((double)d.d);
  return hip_status(sa::launch_block_scores(qbar, kbar, scores, scale, d, (hipStream_t)stream),
                    "block score launch");
}

int32_t sparse_attn_select_f32(const float* scores, const sa_geom* g, double k_frac, double p,
                               const int32_t* row_budget, int32_t* lut, int32_t* counts, int32_t cap,
                               void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(scores, 4, "scores"));
  int kc = 0;
  SA_TRY(check_select_args(d, k_frac, p, row_budget, lut, counts, cap, kc));
  return hip_status(sa::launch_select(scores, d, kc, p, row_budget, lut, counts, cap, (hipStream_t)stream),
                    "select launch");
}

int32_t sparse_attn_select(const double* scores, const sa_geom* g, double k_frac, double p,
                           const int32_t* row_budget, int32_t* lut, int32_t* counts, int32_t cap,
                           void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(scores, 8, "scores"));
  int kc = 0;
  SA_TRY(check_select_args(d, k_frac, p, row_budget, lut, counts, cap, kc));
  return hip_status(sa::launch_select(scores, d, kc, p, row_budget, lut, counts, cap, (hipStream_t)stream),
                    "select launch");
}

size_t sparse_attn_mask_workspace_bytes(const sa_geom* g) {
  sa::Geom d;
  if (make_geom(g, d) != SA_OK) return 0;
  return mask_ws_bytes(d);
}

int32_t sparse_attn_build_mask(const void* qc, const void* kc, const sa_geom* g, int32_t block,
                               double k_frac, double p, const int32_t* row_budget, int32_t* lut,
                               int32_t* counts, int32_t cap, void* workspace, size_t workspace_bytes,
                               void* stream) {
  sa::Geom d;
  int kcount = 0;
  SA_TRY(sa_validate_build_mask(qc, kc, g, block, k_frac, p, row_budget, lut, counts, cap, d, kcount));
  SA_TRY(check_ptr(workspace, kWsAlign, "workspace"));
  const size_t need = mask_ws_bytes(d);
  if (workspace_bytes < need)
    return fail(SA_ERR_CAPACITY, "workspace of %zu bytes is below the %zu needed", workspace_bytes, need);
  const size_t rows = (size_t)d.batch * d.heads * d.nblk;
  char* ws = static_cast<char*>(workspace);
  double* qbar = reinterpret_cast<double*>(ws);
  double* kbar = reinterpret_cast<double*>(ws + round_up(rows * d.d * sizeof(double)));
  float* scores = reinterpret_cast<float*>(ws + 2 * round_up(rows * d.d * sizeof(double)));
  hipStream_t s = (hipStream_t)stream;
  SA_TRY(hip_status(sa::launch_pool(qc, kc, qbar, kbar, d, s), "pool launch"));
  SA_TRY(hip_status(sa::launch_block_scores(qbar, kbar, scores, 1.0 / std::sqrt((double)d.d), d, s),
                    "block score launch"));
  return hip_status(sa::launch_select(scores, d, kcount, p, row_budget, lut, counts, cap, s), "select launch");
}

size_t sparse_attn_mask_groups_workspace_bytes(const sa_geom* g, int32_t qgroup) {
  sa::Geom d;
  int shift = 0;
  if (make_geom(g, d) != SA_OK || check_qgroup(qgroup, shift) != SA_OK) return 0;
  return mask_groups_ws_bytes(d, qgroup);
}

int32_t sparse_attn_build_mask_groups(const void* qc, const void* kc, const sa_geom* g, int32_t qgroup,
                                      double k_frac, double p, int32_t* lut, int32_t* counts, int32_t cap,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  int shift = 0;
  SA_TRY(check_qgroup(qgroup, shift));
  SA_TRY(check_ptr(qc, 16, "qc"));
  SA_TRY(check_ptr(kc, 16, "kc"));
  int kcount = 0;
  SA_TRY(check_select_args(d, k_frac, p, nullptr, lut, counts, cap, kcount));
  SA_TRY(check_ptr(workspace, kWsAlign, "workspace"));
  const size_t need = mask_groups_ws_bytes(d, qgroup);
  if (workspace_bytes < need)
    return fail(SA_ERR_CAPACITY, "workspace of %zu bytes is below the %zu needed", workspace_bytes, need);
  const size_t bh = (size_t)d.batch * d.heads;
  const int nq = (d.nblk + qgroup - 1) / qgroup;
  char* ws = static_cast<char*>(workspace);
  double* qbar = reinterpret_cast<double*>(ws);
  double* kbar = reinterpret_cast<double*>(ws + round_up(bh * nq * d.d * sizeof(double)));
  float* scores = reinterpret_cast<float*>(ws + round_up(bh * nq * d.d * sizeof(double)) +
                                           round_up(bh * d.nblk * d.d * sizeof(double)));
  hipStream_t s = (hipStream_t)stream;
  SA_TRY(hip_status(sa::launch_pool_groups(qc, qbar, qgroup, d, s), "group pool launch"));
  SA_TRY(hip_status(sa::launch_pool_groups(kc, kbar, 1, d, s), "pool launch"));
  SA_TRY(hip_status(sa::launch_block_scores(qbar, kbar, scores, 1.0 / std::sqrt((double)d.d), d, s, nq),
                    "block score launch"));
  return hip_status(sa::launch_select(scores, d, kcount, p, nullptr, lut, counts, cap, s, nq), "select launch");
}

int32_t sparse_attn_fwd_groups(const void* qc, const void* kc, const void* vc, const int32_t* lut,
                               const int32_t* counts, int32_t cap, int32_t qgroup, const sa_geom* g,
                               float scale, void* oc, float* lse_c, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  int shift = 0;
  SA_TRY(check_qgroup(qgroup, shift));
  SA_TRY(check_ptr(qc, 16, "qc"));
  SA_TRY(check_ptr(kc, 16, "kc"));
  SA_TRY(check_ptr(vc, 16, "vc"));
  SA_TRY(check_ptr(lut, 4, "lut"));
  SA_TRY(check_ptr(counts, 4, "counts"));
  SA_TRY(check_ptr(oc, 16, "oc"));
  SA_TRY(check_ptr(lse_c, 4, "lse_c"));
  if (cap < 1) return fail(SA_ERR_INVALID_ARG, "cap must be >= 1");
  if (!std::isfinite(scale)) return fail(SA_ERR_INVALID_ARG, "scale must be finite");
  if (scale <= 0.f) scale = (float)(1.0 / std::sqrt((double)d.d));
  return hip_status(sa::launch_fwd(qc, kc, vc, lut, counts, cap, d, scale, oc, lse_c, nullptr,
                                   (hipStream_t)stream, shift),
                    "fwd launch");
}

size_t sparse_attn_sequence_workspace_bytes(const sa_geom* g) {
  sa::Geom d;
  if (make_geom(g, d) != SA_OK) return 0;
  return sa::sequence_workspace_bytes(d);
}

int32_t sparse_attn_select_per_sequence(const double* scores, const sa_geom* g, double k_frac, int32_t* lut,
                                        int32_t* counts, int32_t cap, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(scores, 8, "scores"));
  if (d.nblk > kMaxSelectBlocks)
    return fail(SA_ERR_UNSUPPORTED, "selection supports at most %d blocks per head (got %d)",
                kMaxSelectBlocks, d.nblk);
  if (!std::isfinite(k_frac)) return fail(SA_ERR_INVALID_ARG, "k_frac must be finite");
  SA_TRY(check_ptr(lut, 4, "lut"));
  SA_TRY(check_ptr(counts, 4, "counts"));
  // a row may win every block: the lists need room for nblk ids
  if (cap < d.nblk) return fail(SA_ERR_CAPACITY, "cap %d is below the largest possible row count %d", cap, d.nblk);
  const int kcount = ceil_k_impl(k_frac, d.nblk);
  SA_TRY(check_ptr(workspace, kWsAlign, "workspace"));
  const size_t need = sa::sequence_workspace_bytes(d);
  if (workspace_bytes < need)
    return fail(SA_ERR_CAPACITY, "workspace of %zu bytes is below the %zu needed", workspace_bytes, need);
  const long long total = (long long)d.nblk * kcount;
  hipStream_t s = (hipStream_t)stream;
  int32_t* budget = nullptr;
  SA_TRY(hip_status(sa::launch_sequence_budget(scores, d, total, workspace, &budget, s), "budget launch"));
  return hip_status(sa::launch_select(scores, d, 0, 0.0, budget, lut, counts, cap, s), "select launch");
}

int32_t sparse_attn_ideal_block_mass(const void* qc, const void* kc, const float* lse_d, const sa_geom* g,
                                     float scale, double* mass, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(qc, 16, "qc"));
  SA_TRY(check_ptr(kc, 16, "kc"));
  SA_TRY(check_ptr(lse_d, 4, "lse_d"));
  SA_TRY(check_ptr(mass, 8, "mass"));
  if (!std::isfinite(scale)) return fail(SA_ERR_INVALID_ARG, "scale must be finite");
  if (scale <= 0.f) scale = (float)(1.0 / std::sqrt((double)d.d));
  return hip_status(sa::launch_ideal_mass(qc, kc, lse_d, d, scale, mass, (hipStream_t)stream), "ideal mass launch");
}

size_t sparse_attn_recall_workspace_bytes(const sa_geom* g) {
  sa::Geom d;
  if (make_geom(g, d) != SA_OK) return 0;
  const size_t rows = (size_t)d.batch * d.heads * d.nblk;
  return round_up(rows * d.nblk * sizeof(int32_t)) + round_up(rows * sizeof(int32_t));
}

int32_t sparse_attn_mask_recall(const double* mass, const int32_t* lut, const int32_t* counts, int32_t cap,
                                const sa_geom* g, double* recall, void* workspace, size_t workspace_bytes,
                                void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  if (d.nblk > kMaxSelectBlocks)
    return fail(SA_ERR_UNSUPPORTED, "selection supports at most %d blocks per head (got %d)",
                kMaxSelectBlocks, d.nblk);
  SA_TRY(check_ptr(mass, 8, "mass"));
  SA_TRY(check_ptr(lut, 4, "lut"));
  SA_TRY(check_ptr(counts, 4, "counts"));
  SA_TRY(check_ptr(recall, 8, "recall"));
  if (cap < 1) return fail(SA_ERR_INVALID_ARG, "cap must be >= 1");
  SA_TRY(check_ptr(workspace, kWsAlign, "workspace"));
  const size_t rows = (size_t)d.batch * d.heads * d.nblk;
  const size_t need = round_up(rows * d.nblk * sizeof(int32_t)) + round_up(rows * sizeof(int32_t));
  if (workspace_bytes < need)
    return fail(SA_ERR_CAPACITY, "workspace of %zu bytes is below the %zu needed", workspace_bytes, need);
  int32_t* top = static_cast<int32_t*>(workspace);
  int32_t* top_counts = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                                   round_up(rows * d.nblk * sizeof(int32_t)));
  hipStream_t s = (hipStream_t)stream;
  // the top list of each row has the row's own count: selection with the counts as budgets
  SA_TRY(hip_status(sa::launch_select(mass, d, 0, 0.0, counts, top, top_counts, d.nblk, s), "select launch"));
  return hip_status(sa::launch_recall(lut, counts, cap, top, d, recall, s), "recall launch");
}

size_t sparse_attn_fwd_workspace_bytes(const sa_geom* g) {
  sa::Geom d;
  if (make_geom(g, d) != SA_OK) return 0;
  return sa::fwd_workspace_bytes(d);
}

int32_t sparse_attn_fwd(const void* qc, const void* kc, const void* vc, const int32_t* lut,
                        const int32_t* counts, int32_t cap, const sa_geom* g, float scale, void* oc,
                        float* lse_c, void* workspace, size_t workspace_bytes, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(qc, 16, "qc"));
  SA_TRY(check_ptr(kc, 16, "kc"));
  SA_TRY(check_ptr(vc, 16, "vc"));
  SA_TRY(check_ptr(lut, 4, "lut"));
  SA_TRY(check_ptr(counts, 4, "counts"));
  SA_TRY(check_ptr(oc, 16, "oc"));
  SA_TRY(check_ptr(lse_c, 4, "lse_c"));
  if (cap < 1) return fail(SA_ERR_INVALID_ARG, "cap must be >= 1");
  if (!std::isfinite(scale)) return fail(SA_ERR_INVALID_ARG, "scale must be finite");
  if (scale <= 0.f) scale = (float)(1.0 / std::sqrt((double)d.d));
  if (workspace != nullptr) {
    SA_TRY(check_ptr(workspace, kWsAlign, "workspace"));
    const size_t need = sa::fwd_workspace_bytes(d);
    if (workspace_bytes < need)
      return fail(SA_ERR_CAPACITY, "workspace of %zu bytes is below the %zu needed", workspace_bytes, need);
  }
  return hip_status(sa::launch_fwd(qc, kc, vc, lut, counts, cap, d, scale, oc, lse_c, workspace,
                                   (hipStream_t)stream),
                    "fwd launch");
}

int32_t sparse_attn_fwd_tokens(const void* qc, const void* kc, const void* vc, const int32_t* lut,
                               const int32_t* counts, int32_t cap, const sa_geom* g, float scale, void* o,
                               float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  sa::Geom d;
  SA_TRY(make_geom(g, d));
  SA_TRY(check_ptr(qc, 16, "qc"));
  SA_TRY(check_ptr(kc, 16, "kc"));
  SA_TRY(check_ptr(vc, 16, "vc"));
  SA_TRY(check_ptr(lut, 4, "lut"));
  SA_TRY(check_ptr(counts, 4, "counts"));
  SA_TRY(check_ptr(o, 16, "o"));
  SA_TRY(check_ptr(lse, 4, "lse"));
  if (cap < 1) return fail(SA_ERR_INVALID_ARG, "cap must be >= 1");
  if (!std::isfinite(scale)) return fail(SA_ERR_INVALID_ARG, "scale must be finite");
  if (scale <= 0.f) scale = (float)(1.0 / std::sqrt((double)d.d));
  if (workspace != nullptr) {
    SA_TRY(check_ptr(workspace, kWsAlign, "workspace"));
    const size_t need = sa::fwd_workspace_bytes(d);
    if (workspace_bytes < need)
      return fail(SA_ERR_CAPACITY, "workspace of %zu bytes is below the %zu needed", workspace_bytes, need);
  }
  return hip_status(sa::launch_fwd_tokens(qc, kc, vc, lut, counts, cap, d, scale, o, lse, (hipStream_t)stream,
                                          workspace),
                    "fwd launch");
}

const char* sparse_attn_last_error(void) { return g_last_error; }

}  // extern "C"
