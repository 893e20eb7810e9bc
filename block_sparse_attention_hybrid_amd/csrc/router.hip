// Fine-grained router (gfx950): sub-cube pooling of Q and K, the router
// attention over all sub-cube keys of a head, and its G x G aggregation into
// block-level scores.
//
// "Improving Video Sparse Attention with Fine-grained Router and Sparse
// Rebasing", section 2.2 (router equations, Figure 2, "Kernel
// Implementation"): Q and K are mean-pooled over sub-cubes of R = rt x rh x rw
// tokens (G = 64 / R sub-cubes per cube), P_hat = Softmax(Q_r K_r^T / sqrt(d))
// is taken over every sub-cube key of the head, and a G x G aggregation gives
// block scores P_r.  As the page describes, the softmax is never materialised:
// one kernel computes the router scores twice, first to accumulate each row's
// log-sum-exp, then to apply the softmax and aggregate.  The aggregation sums
// over the key sub-cubes of a block and averages over the query sub-cubes, so
// rows of P_r are probability rows; sub-cubes that hold only pad slots take no
// part.  The output is log P_r in float64, which the hybrid selection consumes
// like the block scores (its row softmax is P_r itself).  Everything runs in
// float64 (v_mfma_f64_16x16x4f64), so the kept lists can be compared with an
// exact evaluation.
#include "sa_launch.h"
#include "sa_layout.h"

#include <math.h>

#include <type_traits>

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;          // router rows / columns per tile
constexpr int kKc = 16;            // k columns staged per step
constexpr int kLd = kKc + 1;

struct SubCube {
  int rt, rh, rw;   // sub-cube sides
  int gt, gh, gw;   // sub-cubes per cube side
  int G;            // sub-cubes per cube
};

// Real extents (tokens along t, h, w) of block j.
__device__ __forceinline__ void block_extent(const Geom& g, int j, int& et, int& eh, int& ew) {
  int bt, bh, bw;
  block_coords(g, j, bt, bh, bw);
  et = min(g.ct, g.frames - bt * g.ct);
  eh = min(g.ch, g.height - bh * g.ch);
  ew = min(g.cw, g.width - bw * g.cw);
}

// Whether sub-cube a of block j holds at least one real token.
__device__ __forceinline__ bool subcube_present(const Geom& g, const SubCube& sc, int j, int a) {
  int et, eh, ew;
  block_extent(g, j, et, eh, ew);
  const int at = a / (sc.gh * sc.gw), ah = (a / sc.gw) % sc.gh, aw = a % sc.gw;
  return at * sc.rt < et && ah * sc.rh < eh && aw * sc.rw < ew;
}

// One workgroup per (block, batch*head): the G sub-cube means of the block,
// float64 sums of bf16 values over the real slots.
__global__ __launch_bounds__(kThreads) void router_pool_kernel(const bf16* __restrict__ xc,
                                                               double* __restrict__ xr, Geom g,
                                                               SubCube sc) {
  __shared__ float tile[kBlock * 129];
  __shared__ long long tok[kBlock];
  const int i = blockIdx.x;
  const long long bh = blockIdx.y;
  const int d = g.d;
  const bf16* src = xc + (bh * g.n_pad + (long long)i * kBlock) * d;
  if (threadIdx.x < kBlock) tok[threadIdx.x] = slot_token(g, i, threadIdx.x);
  for (int u = threadIdx.x; u < kBlock * d; u += kThreads) {
    const int s = u / d, c = u - s * d;
    tile[s * 129 + c] = (float)src[qk_offset(s, c, d)];
  }
  __syncthreads();
  const int per = kBlock / sc.G;   // tokens per sub-cube
  for (int o = threadIdx.x; o < sc.G * d; o += kThreads) {
    const int a = o / d, c = o - a * d;
    const int at = a / (sc.gh * sc.gw), ah = (a / sc.gw) % sc.gh, aw = a % sc.gw;
    double sum = 0.0;
    int cnt = 0;
    for (int u = 0; u < per; ++u) {
      const int ut = u / (sc.rh * sc.rw), uh = (u / sc.rw) % sc.rh, uw = u % sc.rw;
      const int s = ((at * sc.rt + ut) * g.ch + ah * sc.rh + uh) * g.cw + aw * sc.rw + uw;
      if (tok[s] >= 0) {
        sum += (double)tile[s * 129 + c];
        ++cnt;
      }
    }
    xr[((bh * g.nblk + i) * (long long)sc.G + a) * d + c] = cnt > 0 ? sum / (double)cnt : 0.0;
  }
}

// Router scores of a 64 x 64 tile (rows r0.., columns c0..) into LDS S, in
// float64 (v_mfma_f64_16x16x4f64: accumulator row lane/16 + 4r) or float32
// (v_mfma_f32_16x16x4f32, the means rounded to float32 as they are staged:
// accumulator row 4 (lane/16) + r).
template <typename T>
__device__ __forceinline__ void score_tile(const double* __restrict__ qh, const double* __restrict__ kh,
                                           int nr, int d, int r0, int c0, double scale, T* As,
                                           T* Bs, T* S) {
  using Acc = typename std::conditional<std::is_same<T, double>::value, f64x4, f32x4>::type;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  Acc acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = Acc{0, 0, 0, 0};
  const int lr = threadIdx.x >> 2, lc = (threadIdx.x & 3) * 4;
  const int gi = r0 + lr, gj = c0 + lr;
  const double* qrow = qh + (long long)(gi < nr ? gi : nr - 1) * d + lc;
  const double* krow = kh + (long long)(gj < nr ? gj : nr - 1) * d + lc;
  // the next k step's operands are loaded into registers while this step's
  // products run (rows past nr read a clamped row and are zeroed)
  double an[4], bn[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    an[e] = qrow[e];
    bn[e] = krow[e];
  }
  for (int k0 = 0; k0 < d; k0 += kKc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      As[lr * kLd + lc + e] = gi < nr ? (T)an[e] : (T)0;
      Bs[lr * kLd + lc + e] = gj < nr ? (T)bn[e] : (T)0;
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
  const T sc = (T)scale;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = std::is_same<T, double>::value ? (lane >> 4) + 4 * r : 4 * (lane >> 4) + r;
        const int row = wm * 32 + mt * 16 + rr;
        const int col = wn * 32 + nt * 16 + (lane & 15);
        S[row * (kTile + 1) + col] = acc[mt][nt][r] * sc;
      }
  __syncthreads();
}

__device__ __forceinline__ double exp_of(double x) { return exp(x); }
__device__ __forceinline__ float exp_of(float x) { return __expf(x); }

// One workgroup per (64 router rows, batch*head).  Pass 1: log-sum-exp of
// every row over the present sub-cube keys.  Pass 2: P_hat = exp(S - lse),
// aggregated per (query block, key block) pair of the tile.
// Held to 128 registers and 34 KB of LDS: four workgroups (four waves per
// SIMD) instead of three per compute unit, 5% faster with the same output.
// T = float: the sub-cube scores, their exponentials and the tile in float32
// (the log-sum-exp still accumulates in float64), and log P_r written as
// float32 for the float32 selection.
template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void router_kernel(const double* __restrict__ qr, const double* __restrict__ kr, T* __restrict__ scores,
                   double scale, Geom g, SubCube sc) {
  // the staged operands and the score tile are never live at once (a barrier
  // separates the last operand read of a tile from its score writes, and the
  // last score read from the next tile's staging), so they share LDS
  constexpr int kStage = 2 * kTile * kLd, kScores = kTile * (kTile + 1);
  __shared__ T smem[kStage > kScores ? kStage : kScores];
  T* As = smem;
  T* Bs = smem + kTile * kLd;
  T* S = smem;
  __shared__ double lse[kTile];
  __shared__ unsigned char kpres[kTile];
  const int G = sc.G, n = g.nblk, nr = n * G, d = g.d;
  const int r0 = blockIdx.x * kTile;
  const long long bh = blockIdx.y;
  const double* qh = qr + bh * (long long)nr * d;
  const double* kh = kr + bh * (long long)nr * d;
  const int row = threadIdx.x >> 2, part = threadIdx.x & 3;   // 4 threads per tile row

  // pass 1: online max and sum per row (each thread 16 columns of a tile)
  double m = -INFINITY, l = 0.0;
  for (int c0 = 0; c0 < nr; c0 += kTile) {
    if (threadIdx.x < kTile) {
      const int c = c0 + threadIdx.x;
      kpres[threadIdx.x] = c < nr && subcube_present(g, sc, c / G, c % G);
    }
    score_tile(qh, kh, nr, d, r0, c0, scale, As, Bs, S);
    double tm = -INFINITY;
    for (int e = 0; e < 16; ++e) {
      const int c = part * 16 + e;
      if (kpres[c]) tm = fmax(tm, (double)S[row * (kTile + 1) + c]);
    }
    if (tm > -INFINITY) {
      const double mn = fmax(m, tm);
      double sum = 0.0;
      for (int e = 0; e < 16; ++e) {
        const int c = part * 16 + e;
        if (kpres[c]) sum += exp_of((T)((double)S[row * (kTile + 1) + c] - mn));
      }
      l = (m == -INFINITY ? 0.0 : l * exp(m - mn)) + sum;
      m = mn;
    }
    __syncthreads();
  }
  // combine the 4 partial (m, l) of each row (lanes 4 row .. 4 row + 3)
#pragma unroll
  for (int o = 1; o < 4; o <<= 1) {
    const double mo = __shfl_xor(m, o, kWave), lo = __shfl_xor(l, o, kWave);
    const double mn = fmax(m, mo);
    if (mn > -INFINITY) {
      l = (m == -INFINITY ? 0.0 : l * exp(m - mn)) + (mo == -INFINITY ? 0.0 : lo * exp(mo - mn));
      m = mn;
    }
  }
  if (part == 0) lse[row] = m + log(l);
  __syncthreads();

  // pass 2: aggregate exp(S - lse) per (query block, key block) pair
  const int nb = kTile / G;            // blocks per tile side
  const int i0 = r0 / G;
  for (int c0 = 0; c0 < nr; c0 += kTile) {
    if (threadIdx.x < kTile) {
      const int c = c0 + threadIdx.x;
      kpres[threadIdx.x] = c < nr && subcube_present(g, sc, c / G, c % G);
    }
    score_tile(qh, kh, nr, d, r0, c0, scale, As, Bs, S);
    const int j0 = c0 / G;
    // (a) each router row's mass on each key block of the tile, written over
    //     the first score of that block's column range (in place, one owner)
    for (int u = threadIdx.x; u < kTile * nb; u += kThreads) {
      const int rr = u / nb, bj = u - rr * nb;
      T e = 0;
      for (int b = 0; b < G; ++b) {
        const int cc = bj * G + b;
        if (kpres[cc]) e += exp_of((T)((double)S[rr * (kTile + 1) + cc] - lse[rr]));
      }
      S[rr * (kTile + 1) + bj * G] = e;
    }
    __syncthreads();
    // (b) mean over the present query sub-cubes of each query block
    for (int pr = threadIdx.x; pr < nb * nb; pr += kThreads) {
      const int bi = pr / nb, bj = pr - bi * nb;
      const int i = i0 + bi, j = j0 + bj;
      if (i >= n || j >= n) continue;
      double acc = 0.0;
      int na = 0;
      for (int a = 0; a < G; ++a) {
        if (!subcube_present(g, sc, i, a)) continue;
        ++na;
        acc += S[(bi * G + a) * (kTile + 1) + bj * G];
      }
      scores[(bh * n + i) * (long long)n + j] = (T)log(acc / (double)na);
    }
    __syncthreads();
  }
}

SubCube make_subcube(const Geom& g, int rt, int rh, int rw) {
  SubCube s;
  s.rt = rt;
  s.rh = rh;
  s.rw = rw;
  s.gt = g.ct / rt;
  s.gh = g.ch / rh;
  s.gw = g.cw / rw;
  s.G = s.gt * s.gh * s.gw;
  return s;
}

}  // namespace

hipError_t launch_router_pool(const void* xc, double* xr, const Geom& g, int rt, int rh, int rw, hipStream_t s) {
  dim3 grid(g.nblk, g.batch * g.heads);
  router_pool_kernel<<<grid, kThreads, 0, s>>>(static_cast<const bf16*>(xc), xr, g, make_subcube(g, rt, rh, rw));
  return hipGetLastError();
}

template <typename T>
hipError_t router_t(const double* qr, const double* kr, T* scores, double scale, const Geom& g, int rt, int rh,
                    int rw, hipStream_t s) {
  const SubCube sc = make_subcube(g, rt, rh, rw);
  const long long nr = (long long)g.nblk * sc.G;
  dim3 grid((unsigned)((nr + kTile - 1) / kTile), g.batch * g.heads);
  router_kernel<T><<<grid, kThreads, 0, s>>>(qr, kr, scores, scale, g, sc);
  return hipGetLastError();
}

hipError_t launch_router(const double* qr, const double* kr, double* scores, double scale, const Geom& g,
                         int rt, int rh, int rw, hipStream_t s) {
  return router_t(qr, kr, scores, scale, g, rt, rh, rw, s);
}

hipError_t launch_router(const double* qr, const double* kr, float* scores, double scale, const Geom& g,
                         int rt, int rh, int rw, hipStream_t s) {
  return router_t(qr, kr, scores, scale, g, rt, rh, rw, s);
}

}  // namespace sa
