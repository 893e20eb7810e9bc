// Per-block mean pooling of Q and K (gfx950).
//
// SpargeAttention2 summary page, "Block-Pooled Attention for Efficient Mask
// Construction", step 2 (mean pooling of each query and key block); VSA
// summary page, "The Coarse Stage".  Pad slots of a partial cube are not
// tokens and are skipped; the sum is divided by the block's real-token count.
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

template <int D>
__global__ __launch_bounds__(kThreads) void pool_kernel(const u32x4* __restrict__ qc,
                                                        const u32x4* __restrict__ kc,
                                                        double* __restrict__ qbar,
                                                        double* __restrict__ kbar, Geom g) {
  constexpr int NDS = D / 16;            // 16-dim chunks per 32 tokens
  constexpr int J = kBlock * D / 8 / kThreads;   // 16-byte units per thread
  constexpr int NSLOT = NDS / 4;         // distinct ds values per thread
  const int i = blockIdx.x;
  const long long bh = blockIdx.y;
  const int p = threadIdx.x & 63, h = p >> 5, r = p & 31;
  const int c0 = threadIdx.x >> 6;       // wave index = first ds of this thread
  const uint64_t real = block_real_mask(g, i);
  const long long base = (bh * g.n_pad + (long long)i * kBlock) * (D / 8);
  // unit j of this thread is u = threadIdx + 256 j, in chunk c0 + 4 j:
  // ds = (c0 + 4 j) % NDS (slot j % NSLOT), token 32 ((c0 + 4 j) / NDS) + r
  u32x4 vq[J], vk[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    vq[j] = qc[base + threadIdx.x + kThreads * j];
    vk[j] = kc[base + threadIdx.x + kThreads * j];
  }
  double aq[NSLOT][8], ak[NSLOT][8];
#pragma unroll
  for (int a = 0; a < NSLOT; ++a)
#pragma unroll
    for (int e = 0; e < 8; ++e) aq[a][e] = ak[a][e] = 0.0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int chunk = c0 + 4 * j;
    const int s = 32 * (chunk / NDS) + r;
    if ((real >> s) & 1ull) {
      add_bf16x8(aq[j % NSLOT], vq[j]);
      add_bf16x8(ak[j % NSLOT], vk[j]);
    }
  }
  // Sum over the 32 token residues held by the 32 lanes of each half-wave,
  // as a reduce-scatter: at each butterfly step a lane keeps the half of its
  // values whose index matches its lane bit and adds the partner's copy of
  // that half, so after 5 steps lane r holds the complete sum of value r
  // (31 exchanges instead of 5 per value).  Fixed order: the result does not
  // depend on scheduling (and the sums are exact anyway).
  constexpr int NV = 2 * NSLOT * 8;      // values per lane: [tensor][slot][e]
  double v[NV];
#pragma unroll
  for (int a = 0; a < NSLOT; ++a)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[a * 8 + e] = aq[a][e];
      v[NSLOT * 8 + a * 8 + e] = ak[a][e];
    }
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
  // lane r now holds value index (r / (32 / NV)) -- for NV = 32 that is r,
  // for NV = 16 the pairs (r, r ^ 1) hold the same index r / 2
  const int idx = r / (32 / NV);
  if ((r % (32 / NV)) == 0) {
    const double count = (double)block_real_count(g, i);
    const long long out = (bh * g.nblk + i) * (long long)D;
    const int tensor = idx / (NSLOT * 8), a = (idx / 8) % NSLOT, e = idx % 8;
    const int ds = c0 + 4 * a;
    (tensor == 0 ? qbar : kbar)[out + 16 * ds + 8 * h + e] = v[0] / count;
  }
}

}  // namespace

hipError_t launch_pool(const void* qc, const void* kc, double* qbar, double* kbar,
                       const Geom& g, hipStream_t s) {
  dim3 grid(g.nblk, g.batch * g.heads);
  if (g.d == 128)
    pool_kernel<128><<<grid, kThreads, 0, s>>>(static_cast<const u32x4*>(qc), static_cast<const u32x4*>(kc),
                                               qbar, kbar, g);
  else
    pool_kernel<64><<<grid, kThreads, 0, s>>>(static_cast<const u32x4*>(qc), static_cast<const u32x4*>(kc),
                                              qbar, kbar, g);
  return hipGetLastError();
}

}  // namespace sa
