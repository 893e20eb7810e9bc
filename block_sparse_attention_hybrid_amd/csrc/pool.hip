// Per-block mean pooling of Q and K (gfx950).
//
// SpargeAttention2 summary page, "Block-Pooled Attention for Efficient Mask
// Construction", step 2 (mean pooling of each query and key block); VSA
// summary page, "The Coarse Stage".  Pad slots of a partial cube are not
// tokens and are skipped; the sum is divided by the block's real-token count.
//
// One workgroup per (batch*head, block) reads the block's 64 x d bf16 rows of
// Q and of K once (16-byte lane loads, whole rows per wave) and sums them in
// float64 -- exact for bf16 inputs -- so the pooled vectors are the correctly
// rounded means.  The partial sums of the row groups are combined in LDS in a
// fixed order, so the result does not depend on scheduling.  The kernel is
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

__global__ __launch_bounds__(kThreads) void pool_kernel(const u32x4* __restrict__ qc,
                                                        const u32x4* __restrict__ kc,
                                                        double* __restrict__ qbar,
                                                        double* __restrict__ kbar, Geom g) {
  // row-group partial sums, [tensor][row group * d + column]; groups * d == 2048
  __shared__ double red[2][kThreads * 8];
  const int i = blockIdx.x;
  const long long bh = blockIdx.y;
  const int cpr = g.d / 8;               // 16-byte chunks per row
  const int groups = kThreads / cpr;     // row groups (16 for d=128, 32 for d=64)
  const int c = threadIdx.x % cpr;
  const int rg = threadIdx.x / cpr;
  const uint64_t real = block_real_mask(g, i);
  const long long base = (bh * g.n_pad + (long long)i * kBlock) * cpr + c;
  double aq[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  double ak[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int s = rg; s < kBlock; s += groups) {
    if ((real >> s) & 1ull) {
      add_bf16x8(aq, qc[base + (long long)s * cpr]);
      add_bf16x8(ak, kc[base + (long long)s * cpr]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[0][rg * g.d + c * 8 + e] = aq[e];
    red[1][rg * g.d + c * 8 + e] = ak[e];
  }
  __syncthreads();
  const double count = (double)block_real_count(g, i);
  const long long out = (bh * g.nblk + i) * (long long)g.d;
  for (int t = threadIdx.x; t < 2 * g.d; t += kThreads) {
    const int which = t / g.d, col = t - which * g.d;
    double sum = 0.0;
    for (int r = 0; r < groups; ++r) sum += red[which][r * g.d + col];
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
