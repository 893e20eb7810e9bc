// Host-side launchers of the gfx950 kernels.  Arguments are validated by the
// C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_device.h"

namespace sa {

hipError_t launch_reorder(const void* x, void* xc, int layout, const Geom& g, hipStream_t s);
hipError_t launch_reorder_pool(const void* x, void* xc, int layout, double* xbar, const Geom& g,
                               hipStream_t s);
hipError_t launch_reorder_qkv(const void* q, const void* k, const void* v, void* qc, void* kc, void* vc,
                              double* qbar, double* kbar, const Geom& g, hipStream_t s);
hipError_t launch_unreorder(const void* oc, void* o, const float* lse_c, float* lse,
                            const Geom& g, hipStream_t s);
hipError_t launch_pool(const void* qc, const void* kc, double* qbar, double* kbar,
                       const Geom& g, hipStream_t s);
// Query groups: qg consecutive cubes form one query block (qg = 1: the cube
// itself); a head then has (nblk + qg - 1) / qg query blocks.
hipError_t launch_pool_groups(const void* xc, double* xbar, int qg, const Geom& g, hipStream_t s);
// nrows query rows per head (default nblk) against nblk key blocks
hipError_t launch_block_scores(const double* qbar, const double* kbar, double* scores,
                               double scale, const Geom& g, hipStream_t s, int nrows = -1);
// the same scores written as float32 (three-term bf16 splits on the bf16 matrix cores)
hipError_t launch_block_scores(const double* qbar, const double* kbar, float* scores,
                               double scale, const Geom& g, hipStream_t s, int nrows = -1);
// rows_per_head rows of nblk scores per head (default nblk)
hipError_t launch_select(const double* scores, const Geom& g, int kc_default, double p,
                         const int32_t* row_budget, int32_t* lut, int32_t* counts,
                         int cap, hipStream_t s, int rows_per_head = -1);
// the same selection on float32 scores (each widened exactly to float64)
hipError_t launch_select(const float* scores, const Geom& g, int kc_default, double p,
                         const int32_t* row_budget, int32_t* lut, int32_t* counts,
                         int cap, hipStream_t s, int rows_per_head = -1);
// cube i of a head reads list row i >> qg_shift of its head's nlists rows
// (default: one list per cube).  With a workspace (fwd_workspace_bytes) and
// one list per cube, the rows run in the count-balanced order; without one,
// in the sweep order.  max_count: an upper bound on every list's length that
// the caller knows (-1: none); when it rules out dense groups, the
// dense-group kernel is not launched.
hipError_t launch_fwd(const void* qc, const void* kc, const void* vc, const int32_t* lut,
                      const int32_t* counts, int cap, const Geom& g, float scale, void* oc,
                      float* lse_c, void* workspace, hipStream_t s, int qg_shift = 0, int max_count = -1);
// the forward with the inverse re-indexing fused: O [.., N, d] and LSE [.., N]
// in token order (pad slots not written); workspace and max_count as for
// launch_fwd
hipError_t launch_fwd_tokens(const void* qc, const void* kc, const void* vc, const int32_t* lut,
                             const int32_t* counts, int cap, const Geom& g, float scale, void* o,
                             float* lse, hipStream_t s, void* workspace = nullptr, int max_count = -1);
size_t fwd_workspace_bytes(const Geom& g);
hipError_t launch_router_pool(const void* xc, double* xr, const Geom& g, int rt, int rh, int rw, hipStream_t s);
// workspace NULL: two passes over the sub-cube scores; otherwise one pass with
// its per-block sums in the workspace (>= router_workspace_bytes for one head;
// the heads then run in chunks of what it holds)
hipError_t launch_router(const double* qr, const double* kr, double* scores, double scale, const Geom& g,
                         int rt, int rh, int rw, hipStream_t s, void* workspace = nullptr, size_t ws_bytes = 0);
// the same in float32 (log-sum-exp in float64), log P_r written as float32
hipError_t launch_router(const double* qr, const double* kr, float* scores, double scale, const Geom& g,
                         int rt, int rh, int rw, hipStream_t s, void* workspace = nullptr, size_t ws_bytes = 0);
// bytes of one-pass scratch for `heads` (batch*head) rows of scores of elem bytes
size_t router_workspace_bytes(const Geom& g, int rt, int rh, int rw, size_t elem, int heads);
// Operands of the backward pass (device pointers, see sparse_attn_bwd).
struct BwdArgs {
  const void *q, *k, *v_qk, *k_v, *do_qk;
  const float *lse, *delta;
  const int32_t *lut, *counts;
  int cap;
  const int32_t *lut_t, *counts_t;
  int cap_t;
};
hipError_t launch_bwd_delta(const void* oc, const void* do_qk, float* delta, const Geom& g, hipStream_t s);
size_t transpose_workspace_bytes(const Geom& g);
hipError_t launch_transpose_lut(const int32_t* lut, const int32_t* counts, int cap, int32_t* lut_t,
                                int32_t* counts_t, int cap_t, const Geom& g, void* workspace, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, const Geom& g, float scale, void* dq, void* dk, void* dv, hipStream_t s);
hipError_t launch_pooled_mass(const double* scores, const int32_t* lut, const int32_t* counts, int cap,
                              const Geom& g, double* mass, hipStream_t s);
// rel_drop, rel_ren: Eq. 8's two terms per query block (both NULL: not computed)
hipError_t launch_mask_error(const float* lse_s, const float* lse_d, const void* o_s, const void* o_d,
                             const Geom& g, float* tau, float* rel, hipStream_t s, float* rel_drop = nullptr,
                             float* rel_ren = nullptr);
// Per-sequence Top-K: per-row counts of the head-wide budget `total` over the
// row-softmax of block scores, written to a region of the workspace
// (*budget_out, [batch*heads*nblk] int32).
size_t sequence_workspace_bytes(const Geom& g);
hipError_t launch_sequence_budget(const double* scores, const Geom& g, long long total, void* workspace,
                                  int32_t** budget_out, hipStream_t s);
// P_ideal [batch*heads, nblk, nblk] float64 from a dense run's LSE
hipError_t launch_ideal_mass(const void* qc, const void* kc, const float* lse_d, const Geom& g, float scale,
                             double* mass, hipStream_t s);
// recall per row of kept lists against top lists [batch*heads*nblk, nblk] of the same counts
hipError_t launch_recall(const int32_t* lut, const int32_t* counts, int cap, const int32_t* top, const Geom& g,
                         double* recall, hipStream_t s);
hipError_t launch_coarse(const double* scores, const double* vbar, double* oc, const Geom& g, hipStream_t s);

}  // namespace sa
