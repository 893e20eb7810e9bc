// Pooled block scores S = Qbar Kbar^T * scale on the float64 matrix cores
// (gfx950 v_mfma_f64_16x16x4f64).
//
// SpargeAttention2 summary page, "Block-Pooled Attention for Efficient Mask
// Construction", step 3; VSA2 section 2.2 (coarse branch scores).  The
// contraction is small (2 nblk^2 d flops per head) but decides the kept-block
// lists, so it runs in float64: an fp64 result leaves the selection's order
// decisions to values that differ from an exact evaluation by ~1e-16
// relative, far inside the 1e-6 near-tie margin the lists are checked with.
//
// Tiling: one workgroup of 4 waves computes a 64 x 64 tile of one head's
// scores; each wave owns a 32 x 32 quarter as 2 x 2 MFMA tiles of 16 x 16.
// Operand lanes: A row = lane % 16, B column = lane % 16, k = lane / 16; the
// accumulator's register r of lane l holds row l / 16 + 4 r, column l % 16
// for the float64 product, and row 4 (l / 16) + r, column l % 16 for the
// float32 one.  The k dimension (d) is staged through LDS 16 columns at a
// time; the global loads of the next 16 columns are in flight while the
// current ones are used.
//
// The float32 form (v_mfma_f32_16x16x4f32, twice the float64 matrix rate,
// half the bytes written) rounds the float64 means to float32 when they are
// staged and writes float32 scores: their error is a few 1e-7 of a row's
// largest score, inside the 1e-6 margin at which two scores count as tied.
#include "sa_launch.h"

#include <type_traits>

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kKc = 16;            // k columns staged per step
constexpr int kLd = kKc + 1;       // padded LDS row (doubles)

template <typename T>
__global__ __launch_bounds__(kThreads) void block_scores_kernel(const double* __restrict__ qbar,
                                                                const double* __restrict__ kbar,
                                                                T* __restrict__ scores,
                                                                double scale, Geom g, int nrows) {
  using Acc = typename std::conditional<std::is_same<T, double>::value, f64x4, f32x4>::type;
  __shared__ T As[kTile * kLd];
  __shared__ T Bs[kTile * kLd];
  const int n = g.nblk, d = g.d;   // n key blocks; nrows query rows (n, or n / qg groups)
  const int i0 = blockIdx.y * kTile, j0 = blockIdx.x * kTile;
  const long long bh = blockIdx.z;
  const double* qh = qbar + bh * (long long)nrows * d;
  const double* kh = kbar + bh * (long long)n * d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  Acc acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = Acc{0, 0, 0, 0};

  const int lr = threadIdx.x >> 2;          // tile row this thread stages
  const int lc = (threadIdx.x & 3) * 4;     // first of its 4 columns
  const int gi = i0 + lr, gj = j0 + lr;
  const double* qrow = qh + (long long)(gi < nrows ? gi : nrows - 1) * d + lc;
  const double* krow = kh + (long long)(gj < n ? gj : n - 1) * d + lc;
  // the next step's operands are loaded into registers while this step's
  // products run (rows past n read a clamped row and are zeroed)
  double an[4], bn[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    an[e] = qrow[e];
    bn[e] = krow[e];
  }
  for (int k0 = 0; k0 < d; k0 += kKc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      As[lr * kLd + lc + e] = gi < nrows ? (T)an[e] : (T)0;
      Bs[lr * kLd + lc + e] = gj < n ? (T)bn[e] : (T)0;
    }
    __syncthreads();
    if (k0 + kKc < d) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        an[e] = qrow[k0 + kKc + e];
        bn[e] = krow[k0 + kKc + e];
      }
    }
#pragma unroll
    for (int ks = 0; ks < kKc; ks += 4) {
      const int kk = ks + (lane >> 4);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const T a = As[(wm * 32 + mt * 16 + (lane & 15)) * kLd + kk];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const T b = Bs[(wn * 32 + nt * 16 + (lane & 15)) * kLd + kk];
          if constexpr (std::is_same<T, double>::value)
            acc[mt][nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[mt][nt], 0, 0, 0);
          else
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[mt][nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  T* out = scores + bh * (long long)nrows * n;
  const T sc = (T)scale;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = std::is_same<T, double>::value ? (lane >> 4) + 4 * r : 4 * (lane >> 4) + r;
        const int row = i0 + wm * 32 + mt * 16 + rr;
        const int col = j0 + wn * 32 + nt * 16 + (lane & 15);
        if (row < nrows && col < n) out[(long long)row * n + col] = acc[mt][nt][r] * sc;
      }
}

template <typename T>
hipError_t launch_scores_t(const double* qbar, const double* kbar, T* scores, double scale, const Geom& g,
                           hipStream_t s, int nrows) {
  if (nrows < 0) nrows = g.nblk;
  const int ctiles = (g.nblk + kTile - 1) / kTile, rtiles = (nrows + kTile - 1) / kTile;
  dim3 grid(ctiles, rtiles, g.batch * g.heads);
  block_scores_kernel<T><<<grid, kThreads, 0, s>>>(qbar, kbar, scores, scale, g, nrows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_scores(const double* qbar, const double* kbar, double* scores,
                               double scale, const Geom& g, hipStream_t s, int nrows) {
  return launch_scores_t(qbar, kbar, scores, scale, g, s, nrows);
}

hipError_t launch_block_scores(const double* qbar, const double* kbar, float* scores,
                               double scale, const Geom& g, hipStream_t s, int nrows) {
  return launch_scores_t(qbar, kbar, scores, scale, g, s, nrows);
}

}  // namespace sa
