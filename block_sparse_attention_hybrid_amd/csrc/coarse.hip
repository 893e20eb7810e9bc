// Coarse branch output: attention at block granularity on pooled tokens
// (gfx950, float64 matrix cores).
//
// VSA summary page, "The Coarse Stage": the pooled queries, keys and values of
// the cubes attend to each other, O_c = softmax(Qbar Kbar^T * scale) Vbar, and
// row i of O_c is the coarse output of every token of cube i (VSA2 section 2.2
// keeps the same branch).  The scores S = Qbar Kbar^T * scale are the ones the
// mask is selected from, so this kernel reads them instead of recomputing.
//
// One workgroup of 4 waves owns 64 query blocks of one head.  It first takes
// each row's max m and sum Z of exp(S - m) in float64, then runs the product
// P Vbar over the key blocks in chunks of 16: the chunk's probabilities
// exp(S - m) / Z (float64) and the chunk of Vbar are staged in LDS and fed to
// v_mfma_f64_16x16x4f64; wave w accumulates rows 16 w .. 16 w + 15 across all
// head_dim columns.  Operand lanes: A row = lane % 16, B column = lane % 16,
// k = lane / 16; accumulator register r of lane l holds row l / 16 + 4 r,
// column l % 16.
#include "sa_launch.h"

#include <math.h>

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;          // query blocks per workgroup
constexpr int kKc = 16;            // key blocks per staged chunk
constexpr int kLdA = kKc + 1;      // padded LDS row of the probability tile

template <int D>
__global__ __launch_bounds__(kThreads) void coarse_kernel(const double* __restrict__ scores,
                                                          const double* __restrict__ vbar,
                                                          double* __restrict__ oc, Geom g) {
  constexpr int NT = D / 16;       // 16-column output tiles per wave
  __shared__ double As[kRows * kLdA];
  __shared__ double Bs[kKc * (D + 1)];
  __shared__ double rm[kRows], rz[kRows];
  const int n = g.nblk;
  const int i0 = blockIdx.x * kRows;
  const long long bh = blockIdx.y;
  const double* sh = scores + bh * (long long)n * n;
  const double* vh = vbar + bh * (long long)n * D;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // row max and normaliser of this wave's 16 rows
  for (int rr = 0; rr < 16; ++rr) {
    const int row = i0 + 16 * wave + rr;
    double mx = -INFINITY, z = 0.0;
    if (row < n) {
      const double* srow = sh + (long long)row * n;
      for (int j = lane; j < n; j += 64) mx = fmax(mx, srow[j]);
      mx = wave_max(mx);
      for (int j = lane; j < n; j += 64) z += exp(srow[j] - mx);
      z = wave_sum(z);
    }
    if (lane == 0) {
      rm[16 * wave + rr] = mx;
      rz[16 * wave + rr] = z;
    }
  }
  __syncthreads();

  f64x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f64x4{0.0, 0.0, 0.0, 0.0};

  const int ar = threadIdx.x >> 2, ac = (threadIdx.x & 3) * 4;   // probability staging
  for (int j0 = 0; j0 < n; j0 += kKc) {
    {
      const int row = i0 + ar;
      const double m = rm[ar], z = rz[ar];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + ac + e;
        As[ar * kLdA + ac + e] = (row < n && j < n) ? exp(sh[(long long)row * n + j] - m) / z : 0.0;
      }
    }
    for (int u = threadIdx.x; u < kKc * D; u += kThreads) {
      const int k = u / D, c = u - k * D;
      const int j = j0 + k;
      Bs[k * (D + 1) + c] = j < n ? vh[(long long)j * D + c] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kKc; ks += 4) {
      const int kk = ks + (lane >> 4);
      const double a = As[(16 * wave + (lane & 15)) * kLdA + kk];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const double b = Bs[kk * (D + 1) + 16 * t + (lane & 15)];
        acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  double* out = oc + bh * (long long)n * D;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = i0 + 16 * wave + (lane >> 4) + 4 * r;
      if (row < n) out[(long long)row * D + 16 * t + (lane & 15)] = acc[t][r];
    }
}

}  // namespace

hipError_t launch_coarse(const double* scores, const double* vbar, double* oc, const Geom& g, hipStream_t s) {
  dim3 grid((g.nblk + kRows - 1) / kRows, g.batch * g.heads);
  if (g.d == 128)
    coarse_kernel<128><<<grid, kThreads, 0, s>>>(scores, vbar, oc, g);
  else
    coarse_kernel<64><<<grid, kThreads, 0, s>>>(scores, vbar, oc, g);
  return hipGetLastError();
}

}  // namespace sa
