// Mask-quality diagnostics (gfx950).
//
// SpargeAttention2 summary page, "The Sparse Attention Error Decomposition"
// (Eq. 8, where tau is the dense attention mass the kept keys hold) and Table
// 1's L1 error of the sparse output; VSA summary page on how much attention
// mass the selected cubes capture.
//   * pooled mass: per query block, the block-softmax mass its kept blocks hold;
//   * tau: per query, exp(LSE_sparse - LSE_dense) = the dense softmax mass on
//     the kept real keys (the two LSEs come from sparse_attn_fwd with the
//     kept lists and with every block kept);
//   * relative L1 error per query block: sum |o_s - o| / sum |o| over its real
//     queries, o from the dense run.
#include "sa_launch.h"

#include <math.h>

namespace sa {

namespace {

// One wavefront per row: max and normaliser of the row softmax, then the
// mass on the row's kept ids (float64 throughout).
__global__ __launch_bounds__(64) void pooled_mass_kernel(const double* __restrict__ scores,
                                                         const int32_t* __restrict__ lut,
                                                         const int32_t* __restrict__ counts, int cap, int n,
                                                         double* __restrict__ mass) {
  const long long row = blockIdx.x;
  const int lane = threadIdx.x;
  const double* s = scores + row * (long long)n;
  double mx = -INFINITY;
  for (int j = lane; j < n; j += 64) mx = fmax(mx, s[j]);
  mx = wave_max(mx);
  double z = 0.0;
  for (int j = lane; j < n; j += 64) z += exp(s[j] - mx);
  z = wave_sum(z);
  int cnt = counts[row];
  cnt = cnt < 0 ? 0 : (cnt > cap ? cap : cnt);
  double kept = 0.0;
  for (int e = lane; e < cnt; e += 64) {
    const int j = lut[row * cap + e];
    if (j >= 0 && j < n) kept += exp(s[j] - mx);
  }
  kept = wave_sum(kept);
  if (lane == 0) mass[row] = kept / z;
}

// One wavefront per query block, lane = slot.
__global__ __launch_bounds__(64) void mask_error_kernel(const float* __restrict__ lse_s,
                                                        const float* __restrict__ lse_d,
                                                        const bf16* __restrict__ o_s,
                                                        const bf16* __restrict__ o_d, Geom g,
                                                        float* __restrict__ tau, float* __restrict__ rel) {
  const int i = blockIdx.x;
  const long long bh = blockIdx.y;
  const int s = threadIdx.x, d = g.d;
  const long long slot = bh * g.n_pad + (long long)i * kBlock + s;
  const bool real = slot_token(g, i, s) >= 0;
  const float ld = lse_d[slot], ls = lse_s[slot];
  float t = 0.f;
  if (real && ld > -INFINITY) t = ls > -INFINITY ? expf(ls - ld) : 0.f;
  tau[slot] = t;
  double num = 0.0, den = 0.0;
  if (real) {
    const u32x4* a = reinterpret_cast<const u32x4*>(o_s + slot * d);
    const u32x4* b = reinterpret_cast<const u32x4*>(o_d + slot * d);
    for (int c8 = 0; c8 < d / 8; ++c8) {
      const u32x4 x = a[c8], y = b[c8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = __uint_as_float(x[e] << 16), x1 = __uint_as_float(x[e] & 0xffff0000u);
        const float y0 = __uint_as_float(y[e] << 16), y1 = __uint_as_float(y[e] & 0xffff0000u);
        num += (double)fabsf(x0 - y0) + (double)fabsf(x1 - y1);
        den += (double)fabsf(y0) + (double)fabsf(y1);
      }
    }
  }
  num = wave_sum(num);
  den = wave_sum(den);
  if (s == 0) rel[bh * g.nblk + i] = den > 0.0 ? (float)(num / den) : 0.f;
}

}  // namespace

hipError_t launch_pooled_mass(const double* scores, const int32_t* lut, const int32_t* counts, int cap,
                              const Geom& g, double* mass, hipStream_t s) {
  const long long rows = (long long)g.batch * g.heads * g.nblk;
  pooled_mass_kernel<<<(unsigned)rows, 64, 0, s>>>(scores, lut, counts, cap, g.nblk, mass);
  return hipGetLastError();
}

hipError_t launch_mask_error(const float* lse_s, const float* lse_d, const void* o_s, const void* o_d,
                             const Geom& g, float* tau, float* rel, hipStream_t s) {
  dim3 grid(g.nblk, g.batch * g.heads);
  mask_error_kernel<<<grid, 64, 0, s>>>(lse_s, lse_d, static_cast<const bf16*>(o_s), static_cast<const bf16*>(o_d),
                                        g, tau, rel);
  return hipGetLastError();
}

}  // namespace sa
