// Pooled block scores S = Qbar Kbar^T * scale.
//
// SpargeAttention2 summary page, "Block-Pooled Attention for Efficient Mask
// Construction", step 3; VSA2 section 2.2 (coarse branch scores).  The
// contraction is small (2 nblk^2 d flops per head) but decides the kept-block
// lists, so its rounding must stay far below the 1e-6 relative margin at which
// two scores count as tied.
//
// Float64 form (v_mfma_f64_16x16x4f64): one workgroup of 4 waves computes a
// 64 x 64 tile of one head's scores; each wave owns a 32 x 32 quarter as
// 2 x 2 MFMA tiles of 16 x 16.  Operand lanes: A row = lane % 16, B column =
// lane % 16, k = lane / 16; the accumulator's register r of lane l holds row
// l / 16 + 4 r, column l % 16.  The k dimension (d) is staged through LDS 16
// columns at a time; the global loads of the next 16 columns are in flight
// while the current ones are used.
//
// Float32 form (the path's): every float64 mean (Q's multiplied by the scale
// first) is rounded to float32 and that value split exactly into three bf16
// terms, x_f = x0 + x1 + x2 with |x1| <= 2^-8 |x_f| and |x2| <= 2^-16 |x_f|.
// A product of two means is then the sum of the six term products whose
// orders add to at most 2 (x0 y0; x0 y1, x1 y0; x0 y2, x1 y1, x2 y0), each
// exact in float32, on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16) at 16
// times the float32 matrix rate.  The dropped products are below 2^-23 of
// |x y|, the level of the operands' own rounding to float32.  x0 y0 and the
// five smaller products go to two float32 accumulators, so the small ones are
// not rounded at the magnitude of the large; their float32 sum is the score.
// Measured against float64, the error is a few 1e-7 of a row's largest score.
#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kKc = 16;            // k columns staged per step
constexpr int kLd = kKc + 1;       // padded LDS row (doubles)

__global__ __launch_bounds__(kThreads) void block_scores_kernel(const double* __restrict__ qbar,
                                                                const double* __restrict__ kbar,
                                                                double* __restrict__ scores,
                                                                double scale, Geom g, int nrows) {
  __shared__ double As[kTile * kLd];
  __shared__ double Bs[kTile * kLd];
  const int n = g.nblk, d = g.d;   // n key blocks; nrows query rows (n, or n / qg groups)
  const int i0 = blockIdx.y * kTile, j0 = blockIdx.x * kTile;
  const long long bh = blockIdx.z;
  const double* qh = qbar + bh * (long long)nrows * d;
  const double* kh = kbar + bh * (long long)n * d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  f64x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0, 0, 0, 0};

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
      As[lr * kLd + lc + e] = gi < nrows ? an[e] : 0.0;
      Bs[lr * kLd + lc + e] = gj < n ? bn[e] : 0.0;
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
        const double a = As[(wm * 32 + mt * 16 + (lane & 15)) * kLd + kk];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const double b = Bs[(wn * 32 + nt * 16 + (lane & 15)) * kLd + kk];
          acc[mt][nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[mt][nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  double* out = scores + bh * (long long)nrows * n;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = i0 + wm * 32 + mt * 16 + (lane >> 4) + 4 * r;
        const int col = j0 + wn * 32 + nt * 16 + (lane & 15);
        if (row < nrows && col < n) out[(long long)row * n + col] = acc[mt][nt][r] * scale;
      }
}

// ---------------------------------------------------------------------------
// Float32 scores from three-term bf16 splits.
//
// One workgroup of 4 waves computes a 128 x 128 tile of one head's scores;
// wave (wm, wn) owns the 64 x 64 quarter of rows 64 wm.. and columns 64 wn..
// as 2 x 2 MFMA tiles of 32 x 32.  Per 16-dim step every thread loads 8
// float64 means of Q and 8 of K (pieces of two, below), splits them and
// writes each term to LDS.  The LDS tile of a step holds, for each of Q and
// K, 3 terms x 4 groups of 32 rows as 1 KB chunks in which position
// p = h * 32 + r holds dims 8 h .. +7 of row r: lane l of an MFMA reads its
// operand at position l (row l % 32, dims 8 (l / 32) .. +7).  Two such tiles
// alternate, so one barrier per step separates the writes of step s + 1
// from the reads of step s - 1, and the next step's global loads are in
// flight while this step's products run.  The accumulator's register e of
// lane l holds row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32.

constexpr int kT3 = 128;                 // tile side
constexpr int kGroups = kT3 / 32;        // 32-row operand groups per tile side

typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// two means -> their three bf16 terms, each pair packed (element 0 low).  The
// float32 rounding x_f of a mean is the sum of its terms exactly: x0 is the
// bf16 rounding of x_f, the remainder x_f - x0 (exact in float32) has at most
// 16 significant bits, x1 rounds it to 8, and what is left has at most 8, so
// x2 holds it exactly.  Only the one float64 -> float32 conversion per mean
// runs on the float64 unit.
__device__ __forceinline__ void split_pair(double a, double b, uint32_t& t0, uint32_t& t1, uint32_t& t2) {
  const float fa = (float)a, fb = (float)b;
  t0 = pack2(fa, fb);
  const float ra = fa - __uint_as_float(t0 << 16), rb = fb - __uint_as_float(t0 & 0xffff0000u);
  t1 = pack2(ra, rb);
  t2 = pack2(ra - __uint_as_float(t1 << 16), rb - __uint_as_float(t1 & 0xffff0000u));
}

__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// [operand (Q, K)][term][group][position][word]: one 16-byte operand piece is
// four words of two bf16 each
typedef uint32_t SplitTile[2][3][kGroups][kWave][4];

// Staging: a step's slice of a tile row (16 dims, 128 bytes of float64) is 8
// pieces of two means; thread t takes pieces t + 256 e, e < 4, so one load
// instruction of a wavefront reads 8 whole rows' slices (8 full 128-byte
// lines).  Piece w of a row holds dims 2 w, 2 w + 1: operand position
// (w / 4) * 32 + row % 32 of group row / 32, word w % 4.
constexpr int kPieces = 4;

struct Stager {
  const double* src[kPieces];   // this step's piece of each row (step 0)
  int word[kPieces];            // word index in a SplitTile[op][term] slice

  __device__ __forceinline__ void init(const double* base, long long row0, int rows, int d, int r0, int t) {
#pragma unroll
    for (int e = 0; e < kPieces; ++e) {
      const int q = t + kThreads * e, row = q >> 3, w = q & 7;
      src[e] = base + (row0 + min(r0 + row, rows - 1)) * (long long)d + 2 * w;
      word[e] = ((row >> 5) * kWave + (w >> 2) * 32 + (row & 31)) * 4 + (w & 3);
    }
  }

  __device__ __forceinline__ void load(double2 (&x)[kPieces], int step) const {
#pragma unroll
    for (int e = 0; e < kPieces; ++e) x[e] = *reinterpret_cast<const double2*>(src[e] + 16 * step);
  }

  // Q pieces (op 0) are scaled by `scale` in float64 before their rounding to
  // float32, so the products carry the score's scale
  __device__ __forceinline__ void store(SplitTile& t, int op, const double2 (&x)[kPieces], double scale) const {
    uint32_t* w0 = &t[op][0][0][0][0];
    uint32_t* w1 = &t[op][1][0][0][0];
    uint32_t* w2 = &t[op][2][0][0][0];
#pragma unroll
    for (int e = 0; e < kPieces; ++e) {
      uint32_t a, b, c;
      if (op == 0)
        split_pair(x[e].x * scale, x[e].y * scale, a, b, c);
      else
        split_pair(x[e].x, x[e].y, a, b, c);
      w0[word[e]] = a;
      w1[word[e]] = b;
      w2[word[e]] = c;
    }
  }
};

__device__ __forceinline__ u32x4 operand(const SplitTile& t, int op, int term, int grp, int lane) {
  return *reinterpret_cast<const u32x4*>(&t[op][term][grp][lane][0]);
}

__global__ __launch_bounds__(kThreads) void block_scores_split_kernel(const double* __restrict__ qbar,
                                                                      const double* __restrict__ kbar,
                                                                      float* __restrict__ scores, double scale,
                                                                      Geom g, int nrows) {
  __shared__ SplitTile tiles[2];
  const int n = g.nblk, d = g.d;
  const int i0 = blockIdx.y * kT3, j0 = blockIdx.x * kT3;
  const long long bh = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // rows past the end read a clamped row; their scores are not stored
  Stager sq, sk;
  sq.init(qbar, bh * nrows, nrows, d, i0, t);
  sk.init(kbar, bh * n, n, d, j0, t);

  f32x16 big[2][2], small[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) big[a][b][e] = small[a][b][e] = 0.f;

  double2 xq[kPieces], xk[kPieces];
  sq.load(xq, 0);
  sk.load(xk, 0);
  sq.store(tiles[0], 0, xq, scale);
  sk.store(tiles[0], 1, xk, scale);
  __syncthreads();
  const int steps = d >> 4;
  for (int s = 0; s < steps; ++s) {
    const bool more = s + 1 < steps;
    if (more) {
      sq.load(xq, s + 1);
      sk.load(xk, s + 1);
    }
    const SplitTile& cur = tiles[s & 1];
    u32x4 a[3][2], b[3][2];
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        a[p][m] = operand(cur, 0, p, 2 * wm + m, lane);
        b[p][m] = operand(cur, 1, p, 2 * wn + m, lane);
      }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x16 c = small[mt][nt];
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(a[2][mt]), as_bf8(b[0][nt]), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(a[1][mt]), as_bf8(b[1][nt]), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(a[0][mt]), as_bf8(b[2][nt]), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(a[1][mt]), as_bf8(b[0][nt]), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(a[0][mt]), as_bf8(b[1][nt]), c, 0, 0, 0);
        small[mt][nt] = c;
        big[mt][nt] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(a[0][mt]), as_bf8(b[0][nt]), big[mt][nt], 0, 0, 0);
      }
    if (more) {
      sq.store(tiles[(s + 1) & 1], 0, xq, scale);
      sk.store(tiles[(s + 1) & 1], 1, xk, scale);
    }
    __syncthreads();
  }
  float* out = scores + bh * (long long)nrows * n;
  const int hf = lane >> 5, col0 = j0 + wn * 64 + (lane & 31);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = i0 + wm * 64 + mt * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
      if (row >= nrows) continue;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int col = col0 + nt * 32;
        if (col < n)
          out[(long long)row * n + col] = big[mt][nt][e] + small[mt][nt][e];
      }
    }
}

hipError_t launch_scores_f64(const double* qbar, const double* kbar, double* scores, double scale,
                             const Geom& g, hipStream_t s, int nrows) {
  if (nrows < 0) nrows = g.nblk;
  const int ctiles = (g.nblk + kTile - 1) / kTile, rtiles = (nrows + kTile - 1) / kTile;
  dim3 grid(ctiles, rtiles, g.batch * g.heads);
  block_scores_kernel<<<grid, kThreads, 0, s>>>(qbar, kbar, scores, scale, g, nrows);
  return hipGetLastError();
}

hipError_t launch_scores_split(const double* qbar, const double* kbar, float* scores, double scale, const Geom& g,
                               hipStream_t s, int nrows) {
  if (nrows < 0) nrows = g.nblk;
  const int ctiles = (g.nblk + kT3 - 1) / kT3, rtiles = (nrows + kT3 - 1) / kT3;
  dim3 grid(ctiles, rtiles, g.batch * g.heads);
  block_scores_split_kernel<<<grid, kThreads, 0, s>>>(qbar, kbar, scores, scale, g, nrows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_scores(const double* qbar, const double* kbar, double* scores,
                               double scale, const Geom& g, hipStream_t s, int nrows) {
  return launch_scores_f64(qbar, kbar, scores, scale, g, s, nrows);
}

hipError_t launch_block_scores(const double* qbar, const double* kbar, float* scores,
                               double scale, const Geom& g, hipStream_t s, int nrows) {
  return launch_scores_split(qbar, kbar, scores, scale, g, s, nrows);
}

}  // namespace sa
