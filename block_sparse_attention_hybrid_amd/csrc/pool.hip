// Per-block mean pooling of Q and K (gfx950).
//
// SpargeAttention2 summary page, "Block-Pooled Attention for Efficient Mask
// Construction", step 2 (mean pooling of each query and key block); VSA
// summary page, "The Coarse Stage".  Pad slots of a partial cube are not
// tokens and are skipped; the sum is divided by the block's real-token count.
//
// The grouped form pools queries over query blocks of qg consecutive cubes
// (SpargeAttention2's b_q = 128 against b_kv = 64 is qg = 2): the sums of the
// group's cubes meet in the same accumulators and are divided by the group's
// real-token count.
//
// One workgroup per (batch*head, block) reads the block's 64 x d bf16 values
// of Q and of K once, as whole 1 KB chunks of the QK layout (sa_layout.h),
// and sums them in float64 -- exact for bf16 inputs -- so the pooled vectors
// are the correctly rounded means.  Every thread owns a fixed token residue
// r (mod 32) and half-chunk; the 32 partial sums of each dim are added by a
// cross-lane butterfly, so there is no LDS and no barrier.  The kernel is
// bound by HBM reads of Q and K.
#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void add_bf16x8(double acc[8], const u32x4 v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // bf16 -> fp32 is a 16-bit shift of the bit pattern
    acc[2 * k] += (double)__uint_as_float(v[k] << 16);
    acc[2 * k + 1] += (double)__uint_as_float(v[k] & 0xffff0000u);
  }
}

// NT tensors (Q, or Q and K) pooled over groups of qg cubes (qg = 1: blocks)
template <int D, int NT>
__global__ __launch_bounds__(kThreads) void pool_kernel(const u32x4* __restrict__ qc,
                                                        const u32x4* __restrict__ kc,
                                                        double* __restrict__ qbar,
                                                        double* __restrict__ kbar, Geom g, int qg,
                                                        int ngroups) {
  constexpr int NDS = D / 16;            // 16-dim chunks per 32 tokens
  constexpr int J = kBlock * D / 8 / kThreads;   // 16-byte units per thread
  constexpr int NSLOT = NDS / 4;         // distinct ds values per thread
  const int a = blockIdx.x;              // group (the block itself when qg == 1)
  const long long bh = blockIdx.y;
  const int p = threadIdx.x & 63, h = p >> 5, r = p & 31;
  const int c0 = threadIdx.x >> 6;       // wave index = first ds of this thread
  double acc[NT][NSLOT][8];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int s = 0; s < NSLOT; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[t][s][e] = 0.0;
  const int i_end = min((a + 1) * qg, g.nblk);
  int count = 0;
  for (int i = a * qg; i < i_end; ++i) {
    const uint64_t real = block_real_mask(g, i);
    count += block_real_count(g, i);
    const long long base = (bh * g.n_pad + (long long)i * kBlock) * (D / 8);
    // unit j of this thread is u = threadIdx + 256 j, in chunk c0 + 4 j:
    // ds = (c0 + 4 j) % NDS (slot j % NSLOT), token 32 ((c0 + 4 j) / NDS) + r
    u32x4 v[NT][J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      v[0][j] = qc[base + threadIdx.x + kThreads * j];
      if constexpr (NT == 2) v[NT - 1][j] = kc[base + threadIdx.x + kThreads * j];
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int chunk = c0 + 4 * j;
      const int s = 32 * (chunk / NDS) + r;
      if ((real >> s) & 1ull) {
#pragma unroll
        for (int t = 0; t < NT; ++t) add_bf16x8(acc[t][j % NSLOT], v[t][j]);
      }
    }
  }
  // Sum over the 32 token residues held by the 32 lanes of each half-wave,
  // as a reduce-scatter: at each butterfly step a lane keeps the half of its
  // values whose index matches its lane bit and adds the partner's copy of
  // that half, so after 5 steps lane r holds the complete sum of value
  // r / (32 / NV) (NV - 1 exchanges instead of 5 per value).  Fixed order: the
  // result does not depend on scheduling (and the sums are exact anyway).
  constexpr int NV = NT * NSLOT * 8;     // values per lane: [tensor][slot][e]
  double v[NV];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int s = 0; s < NSLOT; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[(t * NSLOT + s) * 8 + e] = acc[t][s][e];
#pragma unroll
  for (int step = 0; step < 5; ++step) {
    const int o = 16 >> step;            // partner distance
    const int half = NV >> (step + 1);   // values kept after this step (0: plain add)
    const bool up = (r & o) != 0;
    if (half >= 1) {
#pragma unroll
      for (int x = 0; x < half; ++x) {
        const double send = up ? v[x] : v[x + half];
        const double keep = up ? v[x + half] : v[x];
        v[x] = keep + __shfl_xor(send, o, kWave);
      }
    } else {
      v[0] += __shfl_xor(v[0], o, kWave);
    }
  }
  const int idx = r / (32 / NV);
  if ((r % (32 / NV)) == 0) {
    const long long out = (bh * ngroups + a) * (long long)D;
    const int tensor = idx / (NSLOT * 8), s = (idx / 8) % NSLOT, e = idx % 8;
    const int ds = c0 + 4 * s;
    (tensor == 0 ? qbar : kbar)[out + 16 * ds + 8 * h + e] = v[0] / (double)count;
  }
}

}  // namespace

hipError_t launch_pool(const void* qc, const void* kc, double* qbar, double* kbar,
                       const Geom& g, hipStream_t s) {
  dim3 grid(g.nblk, g.batch * g.heads);
  const u32x4* q = static_cast<const u32x4*>(qc);
  const u32x4* k = static_cast<const u32x4*>(kc);
  if (g.d == 128)
    pool_kernel<128, 2><<<grid, kThreads, 0, s>>>(q, k, qbar, kbar, g, 1, g.nblk);
  else
    pool_kernel<64, 2><<<grid, kThreads, 0, s>>>(q, k, qbar, kbar, g, 1, g.nblk);
  return hipGetLastError();
}

hipError_t launch_pool_groups(const void* xc, double* xbar, int qg, const Geom& g, hipStream_t s) {
  const int ngroups = (g.nblk + qg - 1) / qg;
  dim3 grid(ngroups, g.batch * g.heads);
  const u32x4* x = static_cast<const u32x4*>(xc);
  if (g.d == 128)
    pool_kernel<128, 1><<<grid, kThreads, 0, s>>>(x, x, xbar, xbar, g, qg, ngroups);
  else
    pool_kernel<64, 1><<<grid, kThreads, 0, s>>>(x, x, xbar, xbar, g, qg, ngroups);
  return hipGetLastError();
}

}  // namespace sa
