// Coarse branch output: attention at block granularity on pooled tokens
// (gfx950, float64 matrix cores).
//
// VSA summary page, "The Coarse Stage": the pooled queries, keys and values of
// the cubes attend to each other, O_c = softmax(Qbar Kbar^T * scale) Vbar, and
// row i of O_c is the coarse output of every token of cube i (VSA2 section 2.2
// keeps the same branch).  The scores S = Qbar Kbar^T * scale are the ones the
// mask is selected from, so this kernel reads them instead of recomputing.
//
// One workgroup of 4 waves owns 32 query blocks of one head.  It first takes
// each row's max m (float64), then runs the product E Vbar over the key blocks
// in chunks of 16, where E = exp(S - m) is computed once per entry: the chunk
// of E (float64) goes to LDS for the matrix cores and into per-thread partial
// row sums Z at the same time, so O_c = (E Vbar) / Z needs one exponential per
// score.  The chunk's Vbar rows are staged beside it; the next chunk's scores
// and Vbar rows are loaded into registers while the current one is multiplied.
// Wave w accumulates rows 16 (w / 2) .. +15 and columns (D / 2)(w % 2) .. +D/2-1
// on v_mfma_f64_16x16x4f64.  Operand lanes: A row = lane % 16, B column =
// lane % 16, k = lane / 16; accumulator register r of lane l holds row
// l / 16 + 4 r, column l % 16.
#include "sa_launch.h"

#include <math.h>

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 32;          // query blocks per workgroup
constexpr int kKc = 16;            // key blocks per staged chunk
constexpr int kLdA = kKc + 1;      // padded LDS row of the E tile
constexpr int kPer = kRows * kKc / kThreads;   // E entries per thread and chunk (2)

// Held to 128 registers (four waves per SIMD, no spills): the kernel waits
// on its score and Vbar loads and on the per-chunk barriers more than it
// issues, and the extra wave made it 13% faster at 720p with the same output.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void coarse_kernel(const double* __restrict__ scores, const double* __restrict__ vbar, double* __restrict__ oc,
                   Geom g) {
  constexpr int NT = D / 32;       // 16-column output tiles per wave (half the columns)
  constexpr int VP = kKc * D / kThreads;   // Vbar values per thread and chunk
  __shared__ double As[kRows * kLdA];
  __shared__ double Bs[kKc * (D + 1)];
  __shared__ double rm[kRows];
  __shared__ double zpart[kThreads];
  const int n = g.nblk;
  const int i0 = blockIdx.x * kRows;
  const long long bh = blockIdx.y;
  const double* sh = scores + bh * (long long)n * n;
  const double* vh = vbar + bh * (long long)n * D;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rb = wave >> 1, ch = wave & 1;

  // row maxima: wave w takes rows 8 w .. 8 w + 7
  for (int rr = 0; rr < kRows / 4; ++rr) {
    const int lr = 8 * wave + rr, row = i0 + lr;
    double mx = -INFINITY;
    if (row < n) {
      const double* srow = sh + (long long)row * n;
      for (int j = lane; j < n; j += 64) mx = fmax(mx, srow[j]);
      mx = wave_max(mx);
    }
    if (lane == 0) rm[lr] = mx;
  }
  __syncthreads();

  // this thread's E entries: row er, columns ec + 0 .. kPer-1 of each chunk
  const int er = threadIdx.x / (kKc / kPer), ec = (threadIdx.x % (kKc / kPer)) * kPer;
  const int erow = i0 + er;
  const double em = rm[er];
  const double* esrc = sh + (long long)(erow < n ? erow : 0) * n;
  double z = 0.0;                 // partial row sum of this thread's entries
  double sn[kPer], vn[VP];
  auto load_chunk = [&](int j0) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int j = j0 + ec + e;
      sn[e] = (erow < n && j < n) ? esrc[j] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < VP; ++u) {
      const int x = threadIdx.x + kThreads * u, k = x / D, c = x - k * D;
      const int j = j0 + k;
      vn[u] = j < n ? vh[(long long)j * D + c] : 0.0;
    }
  };

  f64x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f64x4{0.0, 0.0, 0.0, 0.0};

  load_chunk(0);
  for (int j0 = 0; j0 < n; j0 += kKc) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      // exp(-inf) = 0 for columns past n and rows past n (their max is -inf too: guarded)
      const double ev = (sn[e] == -INFINITY) ? 0.0 : exp(sn[e] - em);
      z += ev;
      As[er * kLdA + ec + e] = ev;
    }
#pragma unroll
    for (int u = 0; u < VP; ++u) {
      const int x = threadIdx.x + kThreads * u, k = x / D, c = x - k * D;
      Bs[k * (D + 1) + c] = vn[u];
    }
    __syncthreads();
    if (j0 + kKc < n) load_chunk(j0 + kKc);
#pragma unroll
    for (int ks = 0; ks < kKc; ks += 4) {
      const int kk = ks + (lane >> 4);
      const double a = As[(16 * rb + (lane & 15)) * kLdA + kk];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const double b = Bs[kk * (D + 1) + (D / 2) * ch + 16 * t + (lane & 15)];
        acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // Z per row: the kKc / kPer threads of a row add their partials in a fixed order
  zpart[threadIdx.x] = z;
  __syncthreads();
  double* out = oc + bh * (long long)n * D;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lr = 16 * rb + (lane >> 4) + 4 * r, row = i0 + lr;
      if (row < n) {
        double zr = 0.0;
#pragma unroll
        for (int q = 0; q < kKc / kPer; ++q) zr += zpart[lr * (kKc / kPer) + q];
        out[(long long)row * D + (D / 2) * ch + 16 * t + (lane & 15)] = acc[t][r] / zr;
      }
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
