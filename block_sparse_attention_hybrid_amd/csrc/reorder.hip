// Cube re-indexing of video tokens and its inverse (gfx950).
//
// VSA summary page, "Cube Partitioning and Token Re-Indexing": tokens of one
// (ct, ch, cw) cube become one contiguous block; VSA2 section 2.2 applies the
// permutation once at the ends of the transformer and pads each grid side up
// to a multiple of the cube side.
//
// One workgroup per (batch*head, block).  Every destination block is 64 rows
// of d bf16 values written contiguously; the source rows of a cube come in
// runs of cw consecutive tokens.  Each lane moves 16-byte chunks, so a wave
// reads and writes whole 256-byte rows (d = 128) and the traffic is the
// algorithmic minimum: N rows read, n_pad rows written.
#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void reorder_kernel(const u32x4* __restrict__ x,
                                                           u32x4* __restrict__ xc, Geom g) {
  const int i = blockIdx.x;                    // block within the head
  const long long bh = blockIdx.y;             // batch*heads + head
  const int cpr = g.d / 8;                     // 16-byte chunks per row
  const long long src_head = bh * g.n_real * cpr;
  const long long dst_blk = (bh * g.n_pad + (long long)i * kBlock) * cpr;
  for (int idx = threadIdx.x; idx < kBlock * cpr; idx += kThreads) {
    const int s = idx / cpr, c = idx - s * cpr;
    const long long n = slot_token(g, i, s);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n >= 0) v = x[src_head + n * cpr + c];
    xc[dst_blk + idx] = v;
  }
}

__global__ __launch_bounds__(kThreads) void unreorder_kernel(const u32x4* __restrict__ oc,
                                                             u32x4* __restrict__ o,
                                                             const float* __restrict__ lse_c,
                                                             float* __restrict__ lse, Geom g) {
  const int i = blockIdx.x;
  const long long bh = blockIdx.y;
  const int cpr = g.d / 8;
  const long long dst_head = bh * g.n_real * cpr;
  const long long src_blk = (bh * g.n_pad + (long long)i * kBlock) * cpr;
  for (int idx = threadIdx.x; idx < kBlock * cpr; idx += kThreads) {
    const int s = idx / cpr, c = idx - s * cpr;
    const long long n = slot_token(g, i, s);
    if (n >= 0) o[dst_head + n * cpr + c] = oc[src_blk + idx];
  }
  if (lse_c != nullptr && threadIdx.x < kBlock) {
    const int s = threadIdx.x;
    const long long n = slot_token(g, i, s);
    if (n >= 0) lse[bh * g.n_real + n] = lse_c[bh * g.n_pad + (long long)i * kBlock + s];
  }
}

}  // namespace

hipError_t launch_reorder(const void* x, void* xc, const Geom& g, hipStream_t s) {
  dim3 grid(g.nblk, g.batch * g.heads);
  reorder_kernel<<<grid, kThreads, 0, s>>>(static_cast<const u32x4*>(x), static_cast<u32x4*>(xc), g);
  return hipGetLastError();
}

hipError_t launch_unreorder(const void* oc, void* o, const float* lse_c, float* lse,
                            const Geom& g, hipStream_t s) {
  dim3 grid(g.nblk, g.batch * g.heads);
  unreorder_kernel<<<grid, kThreads, 0, s>>>(static_cast<const u32x4*>(oc), static_cast<u32x4*>(o),
                                             lse_c, lse, g);
  return hipGetLastError();
}

}  // namespace sa
