// Cube re-indexing of video tokens and its inverse (gfx950).
//
// VSA summary page, "Cube Partitioning and Token Re-Indexing": tokens of one
// (ct, ch, cw) cube become one contiguous block; VSA2 section 2.2 applies the
// permutation once at the ends of the transformer and pads each grid side up
// to a multiple of the cube side.
//
// One workgroup per (batch*head, block).  The block's 64 source rows (runs of
// cw consecutive tokens) are read with 16-byte lane loads into a token-major
// LDS tile, then written out as 1 KB operand chunks in the QK or V element
// order (see sa_layout.h), so both the reads and the writes are whole-row /
// whole-chunk and the traffic is the algorithmic minimum: N rows read, n_pad
// rows written.  QK chunks are 16-byte rows of the tile; a V chunk lane holds
// 8 tokens of one dim, gathered as 2-byte reads down a tile column (lanes of
// a wave read adjacent columns, so the reads spread over the banks).  Pad
// slots are written as zeros.
//
// The fused form also takes the block's mean over its real tokens from the
// tile while it sits in LDS (SpargeAttention2 summary page, "Block-Pooled
// Attention for Efficient Mask Construction", step 2, for queries and keys;
// VSA summary page, "The Coarse Stage", for values), so pooling costs no
// second pass over the tensor.  The sums are float64 (exact for bf16 inputs)
// divided by the real-token count, the same values as the separate pooling
// kernel.
#include "sa_launch.h"
#include "sa_layout.h"

namespace sa {

namespace {

constexpr int kThreads = 256;

// Row-major token index of every slot of block i (-1 for pad slots), in LDS.
__device__ __forceinline__ void fill_slot_table(const Geom& g, int i, long long* tab) {
  if (threadIdx.x < kBlock) tab[threadIdx.x] = slot_token(g, i, threadIdx.x);
  __syncthreads();
}

// LDS of one block's re-indexing: the token-major tile, the slot table and
// the pooling partial sums
struct ReorderLds {
  // tile[s][c], token-major with row pitch d+8 (16-byte rows), for both layouts
  __attribute__((aligned(16))) uint16_t tile[kBlock * (128 + 8)];
  long long tok[kBlock];
  double part[kThreads];
};

// Block i of (batch*head) bh: token rows -> tile -> operand chunks.
template <bool kV, bool kPool>
__device__ __forceinline__ void reorder_block(const u32x4* __restrict__ x, u32x4* __restrict__ xc,
                                              double* __restrict__ xbar, const Geom& g, int i, long long bh,
                                              ReorderLds& L) {
  uint16_t* tile = L.tile;
  const int d = g.d, cpr = d / 8;
  const int ldq = d + 8;
  const long long src_head = bh * g.n_real * cpr;
  const long long dst_blk = (bh * g.n_pad + (long long)i * kBlock) * cpr;
  fill_slot_table(g, i, L.tok);
  for (int idx = threadIdx.x; idx < kBlock * cpr; idx += kThreads) {
    const int s = idx / cpr, c8 = idx - s * cpr;
    const long long n = L.tok[s];
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n >= 0) v = x[src_head + n * cpr + c8];
    *reinterpret_cast<u32x4*>(&tile[s * ldq + c8 * 8]) = v;
  }
  __syncthreads();
  for (int u = threadIdx.x; u < kBlock * cpr; u += kThreads) {
    const int chunk = u >> 6, p = u & 63, h = p >> 5, r = p & 31;
    u32x4 v;
    if (!kV) {
      const int t32 = chunk / (d / 16), ds = chunk % (d / 16);
      v = *reinterpret_cast<const u32x4*>(&tile[(32 * t32 + r) * ldq + 16 * ds + 8 * h]);
    } else {
      // 8 consecutive tokens of one dim: a column of the tile, packed in pairs
      const int dt = chunk >> 2, ks = chunk & 3;
      const uint16_t* col = &tile[(16 * ks + 8 * h) * ldq + 32 * dt + r];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        v[t] = (uint32_t)col[(2 * t) * ldq] | ((uint32_t)col[(2 * t + 1) * ldq] << 16);
    }
    xc[dst_blk + u] = v;
  }
  if (kPool) {
    // per = kThreads / d threads share a dim, each summing 64 / per slots
    // (pad slots hold zeros); partial sums meet in LDS in a fixed order
    const int per = kThreads / d, c = threadIdx.x % d, grp = threadIdx.x / d;
    const int ns = kBlock / per;
    double acc = 0.0;
    for (int s = grp * ns; s < (grp + 1) * ns; ++s)
      acc += (double)__uint_as_float((uint32_t)tile[s * ldq + c] << 16);
    L.part[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x < d) {
      double sum = 0.0;
      for (int q = 0; q < per; ++q) sum += L.part[q * d + c];
      xbar[(bh * g.nblk + i) * (long long)d + c] = sum / (double)block_real_count(g, i);
    }
  }
}

// One workgroup per (batch*head, block).
template <bool kV, bool kPool>
__global__ __launch_bounds__(kThreads) void reorder_kernel(const u32x4* __restrict__ x,
                                                           u32x4* __restrict__ xc,
                                                           double* __restrict__ xbar, Geom g) {
  __shared__ ReorderLds L;
  reorder_block<kV, kPool>(x, xc, xbar, g, blockIdx.x, blockIdx.y, L);
}

// Queries and keys (with pooling) and values in one launch: grid z = 0, 1, 2.
__global__ __launch_bounds__(kThreads) void reorder_qkv_kernel(const u32x4* __restrict__ q,
                                                               const u32x4* __restrict__ k,
                                                               const u32x4* __restrict__ v,
                                                               u32x4* __restrict__ qc, u32x4* __restrict__ kc,
                                                               u32x4* __restrict__ vc, double* __restrict__ qbar,
                                                               double* __restrict__ kbar, Geom g) {
  __shared__ ReorderLds L;
  if (blockIdx.z == 0)
    reorder_block<false, true>(q, qc, qbar, g, blockIdx.x, blockIdx.y, L);
  else if (blockIdx.z == 1)
    reorder_block<false, true>(k, kc, kbar, g, blockIdx.x, blockIdx.y, L);
  else
    reorder_block<true, false>(v, vc, nullptr, g, blockIdx.x, blockIdx.y, L);
}

__global__ __launch_bounds__(kThreads) void unreorder_kernel(const u32x4* __restrict__ oc,
                                                             u32x4* __restrict__ o,
                                                             const float* __restrict__ lse_c,
                                                             float* __restrict__ lse, Geom g) {
  const int i = blockIdx.x;
  const long long bh = blockIdx.y;
  __shared__ long long tok[kBlock];
  const int cpr = g.d / 8;
  const long long dst_head = bh * g.n_real * cpr;
  const long long src_blk = (bh * g.n_pad + (long long)i * kBlock) * cpr;
  fill_slot_table(g, i, tok);
  for (int idx = threadIdx.x; idx < kBlock * cpr; idx += kThreads) {
    const int s = idx / cpr, c = idx - s * cpr;
    const long long n = tok[s];
    if (n >= 0) o[dst_head + n * cpr + c] = oc[src_blk + idx];
  }
  if (lse_c != nullptr && threadIdx.x < kBlock) {
    const int s = threadIdx.x;
    const long long n = tok[s];
    if (n >= 0) lse[bh * g.n_real + n] = lse_c[bh * g.n_pad + (long long)i * kBlock + s];
  }
}

}  // namespace

hipError_t launch_reorder(const void* x, void* xc, int layout, const Geom& g, hipStream_t s) {
  dim3 grid(g.nblk, g.batch * g.heads);
  const u32x4* src = static_cast<const u32x4*>(x);
  u32x4* dst = static_cast<u32x4*>(xc);
  if (layout == 1)
    reorder_kernel<true, false><<<grid, kThreads, 0, s>>>(src, dst, nullptr, g);
  else
    reorder_kernel<false, false><<<grid, kThreads, 0, s>>>(src, dst, nullptr, g);
  return hipGetLastError();
}

hipError_t launch_reorder_pool(const void* x, void* xc, int layout, double* xbar, const Geom& g,
                               hipStream_t s) {
  dim3 grid(g.nblk, g.batch * g.heads);
  const u32x4* src = static_cast<const u32x4*>(x);
  u32x4* dst = static_cast<u32x4*>(xc);
  if (layout == 1)
    reorder_kernel<true, true><<<grid, kThreads, 0, s>>>(src, dst, xbar, g);
  else
    reorder_kernel<false, true><<<grid, kThreads, 0, s>>>(src, dst, xbar, g);
  return hipGetLastError();
}

hipError_t launch_reorder_qkv(const void* q, const void* k, const void* v, void* qc, void* kc, void* vc,
                              double* qbar, double* kbar, const Geom& g, hipStream_t s) {
  dim3 grid(g.nblk, g.batch * g.heads, 3);
  reorder_qkv_kernel<<<grid, kThreads, 0, s>>>(static_cast<const u32x4*>(q), static_cast<const u32x4*>(k),
                                               static_cast<const u32x4*>(v), static_cast<u32x4*>(qc),
                                               static_cast<u32x4*>(kc), static_cast<u32x4*>(vc), qbar, kbar, g);
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
