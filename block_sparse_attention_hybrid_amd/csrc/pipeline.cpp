// The whole path in one call, optionally overlapped across two streams.
//
// Order of the work (the path of the summary pages: cube re-indexing and
// pooling, pooled scores, hybrid selection, block-sparse forward, inverse
// re-indexing).  With an auxiliary stream the rows are taken in parts for the
// mask phase: the query/key re-indexing of the later parts and the value
// re-indexing (bound by HBM) run there beside the masks (bound by compute) on
// the main stream.  The forward then runs there chunk by chunk while the main
// stream re-indexes the output of the previous chunk; when the caller wants
// no slot-major copy of O and LSE, the forward writes token order itself and
// there is nothing left to re-index.  Events order the two streams; the main
// stream's last work waits for the last work of the auxiliary stream, so the
// caller sees completion on the stream it passed.
#include "../../include/sparse_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
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
                         int32_t head_chunk, bool outputs, sa::Geom& d, int& kcount, float& scale_out);
int32_t sa_hip_status(hipError_t e, const char* what);

namespace {

// Parts the rows are cut into for the mask phase on two streams.
constexpr int kMaskParts = 4;

// Events of one call on two streams: [0] the main stream's first re-indexing,
// [1, parts) the auxiliary stream's re-indexing of part c, [parts] its value
// re-indexing, [parts + 1] the main stream's last mask, then one per forward
// chunk.
struct PhaseEvents {
  std::vector<hipEvent_t>* ev = nullptr;
  int parts = 1;
  hipEvent_t first() const { return (*ev)[0]; }
  hipEvent_t part(int c) const { return (*ev)[c]; }
  hipEvent_t values() const { return (*ev)[parts]; }
  hipEvent_t masks() const { return (*ev)[parts + 1]; }
  hipEvent_t chunk(int c) const { return (*ev)[parts + 2 + c]; }
};

// The mask phase: re-indexing (queries and keys pooled on the way, values),
// block scores and selection.  On one stream, in order.  On two, the rows
// are cut into up to kMaskParts parts: `s` re-indexes the first part's
// queries and keys and then builds each part's mask as soon as its inputs
// are ready, while `a` re-indexes the other parts' queries and keys and then
// the values.  The re-indexing is bound by HBM and the scores and selection
// by compute, so the two overlap; `a` starts once the first part is
// re-indexed, which lets the first mask start early.
hipError_t mask_phase(const sa_path_buffers* b, const sa::Geom& d, int kcount, double p, hipStream_t s,
                      hipStream_t a, bool two, const PhaseEvents& ev) {
  const int rows = d.batch * d.heads;
  const double bscale = 1.0 / std::sqrt((double)d.d);
  const size_t tok = (size_t)d.d;             // elements per token row
  const size_t head_c = (size_t)d.n_pad * tok;
  const size_t head_r = (size_t)d.n_real * tok;
  const size_t nb = (size_t)d.nblk;
  hipError_t e;
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
    float* scores = static_cast<float*>(b->scores) + (size_t)r0 * nb * nb;
    hipError_t r = sa::launch_block_scores(b->qbar + (size_t)r0 * nb * tok, b->kbar + (size_t)r0 * nb * tok,
                                           scores, bscale, gc, st);
    if (r != hipSuccess) return r;
    return sa::launch_select(scores, gc, kcount, p, b->row_budget ? b->row_budget + (size_t)r0 * nb : nullptr,
                             b->lut + (size_t)r0 * nb * b->cap, b->counts + (size_t)r0 * nb, b->cap, st);
  };
  if (!two) {
    if ((e = sa::launch_reorder_qkv(b->q, b->k, b->v, b->qc, b->kc, b->vc, b->qbar, b->kbar, d, s)) != hipSuccess)
      return e;
    return mask(0, rows, s);
  }
  const int parts = ev.parts;
  auto lo = [&](int c) { return (int)((long long)rows * c / parts); };
  if ((e = qk_reorder(lo(0), lo(1) - lo(0), s)) != hipSuccess) return e;
  if ((e = hipEventRecord(ev.first(), s)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(a, ev.first(), 0)) != hipSuccess) return e;
  for (int c = 1; c < parts; ++c) {
    if ((e = qk_reorder(lo(c), lo(c + 1) - lo(c), a)) != hipSuccess) return e;
    if ((e = hipEventRecord(ev.part(c), a)) != hipSuccess) return e;
  }
  if ((e = sa::launch_reorder(b->v, b->vc, 1, d, a)) != hipSuccess) return e;
  if ((e = hipEventRecord(ev.values(), a)) != hipSuccess) return e;
  for (int c = 0; c < parts; ++c) {
    if (c > 0 && (e = hipStreamWaitEvent(s, ev.part(c), 0)) != hipSuccess) return e;
    if ((e = mask(lo(c), lo(c + 1) - lo(c), s)) != hipSuccess) return e;
  }
  return hipEventRecord(ev.masks(), s);
}

int32_t setup(const sa_path_buffers* b, const sa_geom* g, double k_frac, double p, float scale, int32_t head_chunk,
              bool outputs, void* stream, void* aux_stream, sa::Geom& d, int& kcount, float& sc, bool& two,
              int& chunk, int& nchunks, PhaseEvents& ev) {
  const int32_t v = sa_validate_path(b, g, k_frac, p, scale, head_chunk, outputs, d, kcount, sc);
  if (v != SA_OK) return v;
  two = aux_stream != nullptr && aux_stream != stream;
  const int rows = d.batch * d.heads;
  chunk = two ? (head_chunk < rows ? head_chunk : rows) : rows;
  nchunks = (rows + chunk - 1) / chunk;
  ev.parts = rows < kMaskParts ? rows : kMaskParts;
  if (two) {
    const hipError_t e = events_for_current_device((size_t)ev.parts + 2 + nchunks, ev.ev);
    if (e != hipSuccess) return sa_hip_status(e, "event creation");
  }
  return SA_OK;
}

}  // namespace

extern "C" int32_t sparse_attn_mask_path(const sa_path_buffers* b, const sa_geom* g, double k_frac, double p,
                                         void* stream, void* aux_stream) {
  sa::Geom d;
  int kcount = 0, chunk = 0, nchunks = 0;
  float sc = 0.f;
  bool two = false;
  PhaseEvents ev;
  const int32_t v = setup(b, g, k_frac, p, 0.f, 1, false, stream, aux_stream, d, kcount, sc, two, chunk, nchunks, ev);
  if (v != SA_OK) return v;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = mask_phase(b, d, kcount, p, s, (hipStream_t)aux_stream, two, ev);
  if (e != hipSuccess) return sa_hip_status(e, "mask phase");
  // the main stream waits for the values too, so completion is observed on it
  if (two && (e = hipStreamWaitEvent(s, ev.values(), 0)) != hipSuccess) return sa_hip_status(e, "stream wait");
  return SA_OK;
}

extern "C" int32_t sparse_attn_attention(const sa_path_buffers* b, const sa_geom* g, double k_frac, double p,
                                         float scale, int32_t head_chunk, void* stream, void* aux_stream) {
  sa::Geom d;
  int kcount = 0, chunk = 0, nchunks = 0;
  float sc = 0.f;
  bool two = false;
  PhaseEvents ev;
  const int32_t v =
      setup(b, g, k_frac, p, scale, head_chunk, true, stream, aux_stream, d, kcount, sc, two, chunk, nchunks, ev);
  if (v != SA_OK) return v;
  hipStream_t s = (hipStream_t)stream;
  hipStream_t a = two ? (hipStream_t)aux_stream : s;
  const int rows = d.batch * d.heads;
  const size_t tok = (size_t)d.d;
  const size_t head_c = (size_t)d.n_pad * tok;
  const size_t head_r = (size_t)d.n_real * tok;
  const size_t nb = (size_t)d.nblk;
  hipError_t e = mask_phase(b, d, kcount, p, s, a, two, ev);
  if (e != hipSuccess) return sa_hip_status(e, "mask phase");
  // Without row budgets no list is longer than max(kc, pc): the Top-p prefix
  // of a row holds at most ceil(p nblk) blocks, since the largest
  // probabilities average at least 1 / nblk (one more for the rounding of the
  // selection's fixed-point masses).  The forward uses the bound to skip the
  // dense-group kernel when no group can be dense.
  int max_count = -1;
  if (b->row_budget == nullptr) {
    const double pc = p >= 1.0 ? (double)d.nblk : std::ceil(p * (double)d.nblk) + 1.0;
    const double bound = std::max((double)kcount, pc);
    max_count = bound >= (double)d.nblk ? d.nblk : (int)bound;
  }
  // the forward runs on the auxiliary stream after the last mask (the values
  // were re-indexed there already)
  if (two && (e = hipStreamWaitEvent(a, ev.masks(), 0)) != hipSuccess) return sa_hip_status(e, "stream wait");
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
      if ((e = sa::launch_fwd_tokens(qc, kc, vc, lut, counts, b->cap, gc, sc, o, lse, a, fws, max_count)) !=
          hipSuccess)
        return sa_hip_status(e, "fwd launch");
      if (two) {
        if ((e = hipEventRecord(ev.chunk(c), a)) != hipSuccess) return sa_hip_status(e, "event record");
        if ((e = hipStreamWaitEvent(s, ev.chunk(c), 0)) != hipSuccess) return sa_hip_status(e, "stream wait");
      }
      continue;
    }
    char* oc = static_cast<char*>(b->oc) + (size_t)r0 * head_c * 2;
    float* lse_c = b->lse_c + (size_t)r0 * d.n_pad;
    if ((e = sa::launch_fwd(qc, kc, vc, lut, counts, b->cap, gc, sc, oc, lse_c, fws, a, 0, max_count)) !=
        hipSuccess)
      return sa_hip_status(e, "fwd launch");
    if (two) {
      if ((e = hipEventRecord(ev.chunk(c), a)) != hipSuccess) return sa_hip_status(e, "event record");
      if ((e = hipStreamWaitEvent(s, ev.chunk(c), 0)) != hipSuccess) return sa_hip_status(e, "stream wait");
    }
    if ((e = sa::launch_unreorder(oc, o, lse_c, lse, gc, s)) != hipSuccess)
      return sa_hip_status(e, "unreorder launch");
  }
  return SA_OK;
}
