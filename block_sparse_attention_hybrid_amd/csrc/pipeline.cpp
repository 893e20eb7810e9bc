// The whole path in one call, optionally overlapped across two streams.
//
// Order of the work (the path of the summary pages: cube re-indexing and
// pooling, pooled scores, hybrid selection, block-sparse forward, inverse
// re-indexing).  With an auxiliary stream the rows are taken in two parts for
// the first steps: the query/key re-indexing of part B and the value
// re-indexing (bound by HBM) run there beside the mask of part A (bound by
// compute) on the main stream.  The forward then runs there chunk by chunk
// while the main stream re-indexes the output of the previous chunk; when the
// caller wants no slot-major copy of O and LSE, the forward writes token order
// itself and there is nothing left to re-index.  Events order the two streams; the main stream's last work
// waits for the last forward chunk, so the caller sees completion on the
// stream it passed.
#include "../../include/sparse_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <vector>

#include "sa_launch.h"

namespace {

// Events reused across calls: one pool per thread and device (an event
// belongs to the device that was current when it was created).  Re-recording
// an event is safe while an earlier wait on it is still pending: a wait
// refers to the record that preceded it.
struct EventPool {
  int device = -1;
  std::vector<hipEvent_t> ev;
  hipError_t get(size_t n) {
    while (ev.size() < n) {
      hipEvent_t e;
      const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
      if (r != hipSuccess) return r;
      ev.push_back(e);
    }
    return hipSuccess;
  }
};
thread_local std::vector<EventPool> g_pools;

// The current device's pool, holding at least n events.
hipError_t events_for_current_device(size_t n, std::vector<hipEvent_t>*& out) {
  int dev = 0;
  const hipError_t r = hipGetDevice(&dev);
  if (r != hipSuccess) return r;
  for (EventPool& p : g_pools)
    if (p.device == dev) {
      out = &p.ev;
      return p.get(n);
    }
  g_pools.push_back(EventPool{});
  g_pools.back().device = dev;
  out = &g_pools.back().ev;
  return g_pools.back().get(n);
}

// Geometry of rows [r0, r0 + nr) of the flattened batch*heads dimension.
sa::Geom rows_of(const sa::Geom& d, int nr) {
  sa::Geom s = d;
  s.batch = 1;
  s.heads = nr;
  return s;
}

}  // namespace

// defined in capi.cpp
int32_t sa_validate_path(const sa_path_buffers* b, const sa_geom* g, double k_frac, double p, float scale,
                         int32_t head_chunk, sa::Geom& d, int& kcount, float& scale_out);
int32_t sa_hip_status(hipError_t e, const char* what);

extern "C" int32_t sparse_attn_attention(const sa_path_buffers* b, const sa_geom* g, double k_frac, double p,
                                         float scale, int32_t head_chunk, void* stream, void* aux_stream) {
  sa::Geom d;
  int kcount = 0;
  float sc = 0.f;
  const int32_t v = sa_validate_path(b, g, k_frac, p, scale, head_chunk, d, kcount, sc);
  if (v != SA_OK) return v;
  hipStream_t s = (hipStream_t)stream;
  hipStream_t a = aux_stream != nullptr ? (hipStream_t)aux_stream : s;
  const bool two = aux_stream != nullptr && aux_stream != stream;
  const int rows = d.batch * d.heads;
  const int chunk = two ? (head_chunk < rows ? head_chunk : rows) : rows;
  const int nchunks = (rows + chunk - 1) / chunk;
  const double bscale = 1.0 / std::sqrt((double)d.d);
  const size_t tok = (size_t)d.d;             // elements per token row
  const size_t head_c = (size_t)d.n_pad * tok;
  const size_t head_r = (size_t)d.n_real * tok;
  const size_t nb = (size_t)d.nblk;
  hipError_t e;
  std::vector<hipEvent_t>* evp = nullptr;   // this device's events (two-stream form only)
  // the query and key reorders (with pooling) and the mask of rows [r0, r0 + nr)
  auto qk_reorder = [&](int r0, int nr, hipStream_t st) -> hipError_t {
    const sa::Geom gc = rows_of(d, nr);
    hipError_t r = sa::launch_reorder_pool(static_cast<const char*>(b->q) + (size_t)r0 * head_r * 2,
                                           static_cast<char*>(b->qc) + (size_t)r0 * head_c * 2, 0,
                                           b->qbar + (size_t)r0 * nb * tok, gc, st);
    if (r != hipSuccess) return r;
    return sa::launch_reorder_pool(static_cast<const char*>(b->k) + (size_t)r0 * head_r * 2,
                                   static_cast<char*>(b->kc) + (size_t)r0 * head_c * 2, 0,
                                   b->kbar + (size_t)r0 * nb * tok, gc, st);
  };
  auto mask = [&](int r0, int nr, hipStream_t st) -> hipError_t {
    const sa::Geom gc = rows_of(d, nr);
    double* scores = b->scores + (size_t)r0 * nb * nb;
    hipError_t r = sa::launch_block_scores(b->qbar + (size_t)r0 * nb * tok, b->kbar + (size_t)r0 * nb * tok,
                                           scores, bscale, gc, st);
    if (r != hipSuccess) return r;
    return sa::launch_select(scores, gc, kcount, p, b->row_budget ? b->row_budget + (size_t)r0 * nb : nullptr,
                             b->lut + (size_t)r0 * nb * b->cap, b->counts + (size_t)r0 * nb, b->cap, st);
  };
  if (!two) {
    if ((e = qk_reorder(0, rows, s)) != hipSuccess) return sa_hip_status(e, "reorder_pool launch");
    if ((e = sa::launch_reorder(b->v, b->vc, 1, d, s)) != hipSuccess) return sa_hip_status(e, "reorder launch");
    if ((e = mask(0, rows, s)) != hipSuccess) return sa_hip_status(e, "mask launch");
  } else {
    // Rows are taken in two parts.  The main stream re-indexes part A's
    // queries and keys and builds its mask while the auxiliary stream
    // re-indexes part B's; the main stream then builds part B's mask while the
    // auxiliary stream re-indexes the values (the re-indexing is bound by HBM,
    // the scores and selection by compute).
    const int part = rows > 1 ? rows / 2 : rows;
    if ((e = events_for_current_device(nchunks + 3, evp)) != hipSuccess) return sa_hip_status(e, "event creation");
    if ((e = qk_reorder(0, part, s)) != hipSuccess) return sa_hip_status(e, "reorder_pool launch");
    if ((e = hipEventRecord((*evp)[0], s)) != hipSuccess) return sa_hip_status(e, "event record");
    if ((e = hipStreamWaitEvent(a, (*evp)[0], 0)) != hipSuccess) return sa_hip_status(e, "stream wait");
    if (rows > part && (e = qk_reorder(part, rows - part, a)) != hipSuccess)
      return sa_hip_status(e, "reorder_pool launch");
    if ((e = hipEventRecord((*evp)[1], a)) != hipSuccess) return sa_hip_status(e, "event record");
    if ((e = sa::launch_reorder(b->v, b->vc, 1, d, a)) != hipSuccess) return sa_hip_status(e, "reorder launch");
    if ((e = mask(0, part, s)) != hipSuccess) return sa_hip_status(e, "mask launch");
    if ((e = hipStreamWaitEvent(s, (*evp)[1], 0)) != hipSuccess) return sa_hip_status(e, "stream wait");
    if (rows > part && (e = mask(part, rows - part, s)) != hipSuccess) return sa_hip_status(e, "mask launch");
    if ((e = hipEventRecord((*evp)[2], s)) != hipSuccess) return sa_hip_status(e, "event record");
    if ((e = hipStreamWaitEvent(a, (*evp)[2], 0)) != hipSuccess) return sa_hip_status(e, "stream wait");
  }
  // the forward chunk by chunk on the auxiliary stream; each chunk's output is
  // re-indexed on the main stream while the next chunk's forward runs (the
  // re-indexing kernel is small enough to share the compute units with it).
  // With per-row budgets the rows' list lengths spread widely, and the forward
  // takes its rows in the count-balanced order; the scores are no longer
  // needed once the lists exist, so their buffer holds that order (the chunks
  // run one after another on one stream, so they can share it).
  for (int c = 0; c < nchunks; ++c) {
    const int r0 = c * chunk, nr = (rows - r0) < chunk ? (rows - r0) : chunk;
    const sa::Geom gc = rows_of(d, nr);
    void* fws = b->row_budget != nullptr && (size_t)rows * nb * nb * sizeof(double) >= sa::fwd_workspace_bytes(gc)
                    ? (void*)b->scores
                    : nullptr;
    const int32_t* lut = b->lut + (size_t)r0 * nb * b->cap;
    const int32_t* counts = b->counts + (size_t)r0 * nb;
    const char* qc = static_cast<const char*>(b->qc) + (size_t)r0 * head_c * 2;
    const char* kc = static_cast<const char*>(b->kc) + (size_t)r0 * head_c * 2;
    const char* vc = static_cast<const char*>(b->vc) + (size_t)r0 * head_c * 2;
    char* o = static_cast<char*>(b->o) + (size_t)r0 * head_r * 2;
    float* lse = b->lse + (size_t)r0 * d.n_real;
    if (b->oc == nullptr) {
      // no slot-major copy wanted: the forward writes token order itself
      if ((e = sa::launch_fwd_tokens(qc, kc, vc, lut, counts, b->cap, gc, sc, o, lse, a, fws)) != hipSuccess)
        return sa_hip_status(e, "fwd launch");
      if (two) {
        if ((e = hipEventRecord((*evp)[3 + c], a)) != hipSuccess) return sa_hip_status(e, "event record");
        if ((e = hipStreamWaitEvent(s, (*evp)[3 + c], 0)) != hipSuccess)
          return sa_hip_status(e, "stream wait");
      }
      continue;
    }
    char* oc = static_cast<char*>(b->oc) + (size_t)r0 * head_c * 2;
    float* lse_c = b->lse_c + (size_t)r0 * d.n_pad;
    if ((e = sa::launch_fwd(qc, kc, vc, lut, counts, b->cap, gc, sc, oc, lse_c, fws, a)) != hipSuccess)
      return sa_hip_status(e, "fwd launch");
    if (two) {
      if ((e = hipEventRecord((*evp)[3 + c], a)) != hipSuccess) return sa_hip_status(e, "event record");
      if ((e = hipStreamWaitEvent(s, (*evp)[3 + c], 0)) != hipSuccess) return sa_hip_status(e, "stream wait");
    }
    if ((e = sa::launch_unreorder(oc, o, lse_c, lse, gc, s)) != hipSuccess)
      return sa_hip_status(e, "unreorder launch");
  }
  return SA_OK;
}
