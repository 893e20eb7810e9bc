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
// r (mod 32) and half-chunk; the 32 partial sums of each dim are then added in
// LDS in a fixed order, so the result does not depend on scheduling.  The
// kernel is bound by HBM reads of Q and K.
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

__global__ __launch_bounds__(kThreads) void pool_kernel(const u32x4* __restrict__ qc,
                                                        const u32x4* __restrict__ kc,
                                                        double* __restrict__ qbar,
                                                        double* __restrict__ kbar, Geom g) {
  __shared__ double part[2][32 * 128];   // [tensor][token residue r][dim]
  const int i = blockIdx.x;
  const long long bh = blockIdx.y;
  const int d = g.d, nds = d / 16;
  const int units = kBlock * d / 8;      // 16-byte units per block
  const int p = threadIdx.x & 63, h = p >> 5, r = p & 31;
  const uint64_t real = block_real_mask(g, i);
  const long long base = (bh * g.n_pad + (long long)i * kBlock) * (d / 8);
  // this thread's units: chunk = threadIdx/64 + 4 j; the ds values it meets
  // are chunk % nds, each for tokens r and 32 + r
  double aq[2][8], ak[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int e = 0; e < 8; ++e) aq[a][e] = ak[a][e] = 0.0;
  for (int u = threadIdx.x; u < units; u += kThreads) {
    const int chunk = u >> 6;
    const int t32 = chunk / nds, ds = chunk % nds;
    const int s = 32 * t32 + r;
    const int slot = (ds >> 2) & 1;      // ds = threadIdx/64 (+4): two slots at d = 128
    if ((real >> s) & 1ull) {
      add_bf16x8(aq[slot], qc[base + u]);
      add_bf16x8(ak[slot], kc[base + u]);
    }
  }
  const int c0 = threadIdx.x >> 6;       // first ds of this thread
  for (int slot = 0; slot < 2; ++slot) {
    const int ds = c0 + 4 * slot;
    if (ds >= nds) break;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      part[0][r * 128 + 16 * ds + 8 * h + e] = aq[slot][e];
      part[1][r * 128 + 16 * ds + 8 * h + e] = ak[slot][e];
    }
  }
  __syncthreads();
  const double count = (double)block_real_count(g, i);
  const long long out = (bh * g.nblk + i) * (long long)d;
  for (int t = threadIdx.x; t < 2 * d; t += kThreads) {
    const int which = t / d, col = t - which * d;
    double sum = 0.0;
    for (int rr = 0; rr < 32; ++rr) sum += part[which][rr * 128 + col];
    (which == 0 ? qbar : kbar)[out + col] = sum / count;
  }
}

}  // namespace

hipError_t launch_pool(const void* qc, const void* kc, double* qbar, double* kbar,
                       const Geom& g, hipStream_t s) {
  dim3 grid(g.nblk, g.batch * g.heads);
  pool_kernel<<<grid, kThreads, 0, s>>>(static_cast<const u32x4*>(qc), static_cast<const u32x4*>(kc),
                                        qbar, kbar, g);
  return hipGetLastError();
}

}  // namespace sa
