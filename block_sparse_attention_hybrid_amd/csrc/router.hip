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

#include <algorithm>
#include <type_traits>

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;          // router rows / columns per tile
constexpr int kKc = 16;            // k columns staged per step
constexpr int kSPitch32 = kTile + 4; // float32 score tile pitch of the one-pass kernel
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

// The float32 tile engine of the one-pass kernel.
//
// The sub-cube scores come from exact three-term bf16 splits on the bf16
// matrix cores: every float64 mean (Q's times the scale) is rounded to
// float32 and that value split exactly into x0 + x1 + x2 (each the bf16
// rounding of what the previous terms leave; |x1| <= 2^-8 |x|, |x2| <= 2^-16
// |x|).  A score is the sum of the six term products of order <= 2, each
// exact in float32, on v_mfma_f32_16x16x32_bf16 (16 times the float32 matrix
// rate); the dropped products are below 2^-23 of |x y|, the level of the
// operands' own float32 rounding.  x0 y0 and the five smaller products go to
// two float32 accumulators, whose float32 sum is the score.
//
// K's terms are laid out by a pre-pass so that one wavefront load moves 1 KB
// of consecutive bytes: per (batch*head) and column tile t, 3 D / 8 chunks c =
// term * (D / 8) + k8, each holding for the tile's 64 columns in turn the 8
// bf16 of that term for k = 8 k8 .. +7 (zeros past the last sub-cube).  The
// kernel loads the next tile's share into registers while the current tile
// is multiplied and its softmax taken, and writes it into LDS at the next
// tile's start: [term][column][k], a column's row padded to D + 8 bf16.
//
// Q's terms stay in registers for the whole sweep.  Wave w computes router
// rows 16w .. 16w + 15 of the tile against its 64 columns; product j of lane
// l takes k = 32j + 8 (l >> 4) .. +7 of row 16w + (l & 15) for A and of
// column (l & 15) of each 16-column group for B; the accumulator's register r
// holds row 4 (l >> 4) + r, column l & 15.
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// two values -> their three bf16 terms, each pair packed (element 0 low): the
// float32 rounding of each is the exact sum of its terms
__device__ __forceinline__ void split_pair(double a, double b, uint32_t& t0, uint32_t& t1, uint32_t& t2) {
  const float fa = (float)a, fb = (float)b;
  t0 = pack2(fa, fb);
  const float ra = fa - __uint_as_float(t0 << 16), rb = fb - __uint_as_float(t0 & 0xffff0000u);
  t1 = pack2(ra, rb);
  t2 = pack2(ra - __uint_as_float(t1 << 16), rb - __uint_as_float(t1 & 0xffff0000u));
}

__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// the 8 values at p, scaled, as three u32x4 of bf16 terms
__device__ __forceinline__ void split8(const double* p, double scale, u32x4& w0, u32x4& w1, u32x4& w2) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t a, b, c;
    split_pair(p[2 * e] * scale, p[2 * e + 1] * scale, a, b, c);
    w0[e] = a;
    w1[e] = b;
    w2[e] = c;
  }
}

// One thread per (column tile, 8 k values, column): its three term chunks.
__global__ __launch_bounds__(kThreads) void router_k32_kernel(const double* __restrict__ kr, u32x4* __restrict__ kt,
                                                              int nr, int d, int ntile, int bh0) {
  const int k8n = d / 8;
  const long long per_head = (long long)ntile * k8n * kTile;   // threads (and chunks per term)
  const long long u = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (u >= per_head) return;
  const int bhc = blockIdx.y;
  const int col = (int)(u & 63), k8 = (int)((u >> 6) % k8n), t = (int)((u >> 6) / k8n);
  const int j = t * kTile + col;
  u32x4 w0 = {0, 0, 0, 0}, w1 = w0, w2 = w0;
  if (j < nr) split8(kr + ((long long)(bh0 + bhc) * nr + j) * d + 8 * k8, 1.0, w0, w1, w2);
  u32x4* dst = kt + (long long)bhc * per_head * 3 + ((long long)t * 3 * k8n) * kTile + col;
  dst[(0 * k8n + k8) * kTile] = w0;
  dst[(1 * k8n + k8) * kTile] = w1;
  dst[(2 * k8n + k8) * kTile] = w2;
}

template <int D>
__device__ __forceinline__ void load_q_operands(const double* __restrict__ qh, int nr, int r0, double scale,
                                                u32x4 (&aq)[3][D / 32]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gi = r0 + wave * 16 + (lane & 15);
  const double* qrow = qh + (long long)(gi < nr ? gi : nr - 1) * D + 8 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    split8(qrow + 32 * j, gi < nr ? scale : 0.0, aq[0][j], aq[1][j], aq[2][j]);
  }
}

// This thread's share of column tile t of kt: chunks c = 4i + wave, column
// lane, for i < 3 D / 32.
template <int D>
__device__ __forceinline__ void load_k_share(const u32x4* __restrict__ kth, int t, u32x4 (&kv)[3 * D / 32]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const u32x4* src = kth + (long long)t * 3 * (D / 8) * kTile;
#pragma unroll
  for (int i = 0; i < 3 * D / 32; ++i) kv[i] = src[(4 * i + wave) * 64 + lane];
}

template <int D>
__device__ __forceinline__ void store_k_share(const u32x4 (&kv)[3 * D / 32], __bf16* Ks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 3 * D / 32; ++i) {
    const int c = 4 * i + wave, term = c / (D / 8), k8 = c % (D / 8);
    *reinterpret_cast<u32x4*>(Ks + (term * kTile + lane) * (D + 8) + 8 * k8) = kv[i];
  }
}

// Scores of the tile from the staged K terms (LDS) into S (pitch kSPitch32:
// 4 mod 64 floats, so a wavefront's writes of four rows by 16 columns hit 64
// different banks, and 16-byte aligned rows for the 16-byte reads of a
// thread's 16 columns).
// Ends with a barrier; the caller's barrier before it ordered the K writes.
template <int D>
__device__ __forceinline__ void score_tile_f32(const u32x4 (&aq)[3][D / 32], const __bf16* Ks, float* S) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x4 big[4], small[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) big[nt] = small[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const __bf16* kb = Ks + (nt * 16 + (lane & 15)) * (D + 8) + 32 * j + 8 * (lane >> 4);
      u32x4 b[3];
#pragma unroll
      for (int tb = 0; tb < 3; ++tb) b[tb] = *reinterpret_cast<const u32x4*>(kb + tb * kTile * (D + 8));
      f32x4 c = small[nt];
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(aq[2][j]), as_bf8(b[0]), c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(aq[1][j]), as_bf8(b[1]), c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(aq[0][j]), as_bf8(b[2]), c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(aq[1][j]), as_bf8(b[0]), c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(aq[0][j]), as_bf8(b[1]), c, 0, 0, 0);
      small[nt] = c;
      big[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(aq[0][j]), as_bf8(b[0]), big[nt], 0, 0, 0);
    }
  }
  __syncthreads();   // the staged K is dead; S takes its place
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[(wave * 16 + 4 * (lane >> 4) + r) * kSPitch32 + nt * 16 + (lane & 15)] = big[nt][r] + small[nt][r];
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

__device__ __forceinline__ float larger(float a, float b) { return a > b ? a : b; }
__device__ __forceinline__ double larger(double a, double b) { return a > b ? a : b; }

// Sums of a thread's 16 consecutive exponentials over key blocks of GG
// sub-cubes (GG <= 16: 16 / GG whole blocks), written to dst in order.
template <int GG, typename T>
__device__ __forceinline__ void fold_blocks(const T (&v)[16], T* __restrict__ dst) {
#pragma unroll
  for (int bj = 0; bj < 16 / GG; ++bj) {
    T e = 0;
#pragma unroll
    for (int b = 0; b < GG; ++b) e += v[bj * GG + b];
    dst[bj] = e;
  }
}

// Bit c of word t: sub-cube 64 t + c of a head holds a real token (the same
// for every head).  One wavefront per word.
__global__ __launch_bounds__(kThreads) void router_present_kernel(unsigned long long* __restrict__ pmask, Geom g,
                                                                  SubCube sc, int nr) {
  const int c = blockIdx.x * kThreads + threadIdx.x;
  const bool p = c < nr && subcube_present(g, sc, c / sc.G, c % sc.G);
  const unsigned long long w = __ballot(p);
  if ((threadIdx.x & 63) == 0 && c < ((nr + kTile - 1) / kTile) * kTile) pmask[c >> 6] = w;
}

// One pass over the sub-cube scores instead of two, for callers that give the
// router a scratch buffer.  The page's kernel recomputes every score in a
// second pass because the row log-sum-exp is known only at the end of the
// first; here each row's mass on each key block is kept instead, relative to
// the row's running maximum at the time:
//   E[row][j] = sum over the present sub-cubes b of key block j of
//               exp(S[row][(j, b)] - m_t(row)),
// with m_t(row) the running maximum after column tile t (the tile holding
// j's sub-cubes).  E and m_t go to the scratch buffer; once the sweep has
// passed every column, the log-sum-exp is known and
//   P_hat summed over key block j = exp(m_t(row) - lse(row)) * E[row][j],
// which the G x G aggregation then averages over the query sub-cubes.  So the
// matrix products and the exponentials are computed once instead of twice.
//
// Scratch per (batch*head) of a chunk, for row tile x and column tile t:
//   esum[((x * ntile) + t) * 64 * nb + row * nb + jb]   (nb = 64 / G blocks)
//   emax[((x * ntile) + t) * 64 + row]
// The float32 kernel at two waves per SIMD (168 registers at three spill;
// 10.6 against 11.0 ms at 720p)
#ifndef SA_ROUTER_F32_WAVES
#define SA_ROUTER_F32_WAVES 2
#endif
template <typename T, int D>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(std::is_same<T, double>::value ? 4 : SA_ROUTER_F32_WAVES)))
void router_onepass_kernel(const double* __restrict__ qr, const double* __restrict__ kr, T* __restrict__ scores,
                           T* __restrict__ esum, T* __restrict__ emax, const u32x4* __restrict__ kt,
                           const unsigned long long* __restrict__ pmask, double scale, Geom g, SubCube sc,
                           int bh0) {
  // float32: the engine above (Q in registers, K from kt, a whole tile staged
  // at once); float64, whose operands would take twice the registers: both
  // operands staged 16 k columns at a time (score_tile)
  constexpr bool kF32 = !std::is_same<T, double>::value;
  constexpr int kStage = kF32 ? 3 * kTile * (D + 8) * 2 / (int)sizeof(T) : 2 * kTile * kLd;
  constexpr int kSP = kF32 ? kSPitch32 : kTile + 1;   // score tile pitch
  constexpr int kScores = kTile * kSP;
  constexpr int kCt = 16;   // column tiles per aggregation step
  // the aggregation's rescaling factors reuse the staging area
  constexpr int kWords = ((kStage > kScores ? kStage : kScores) * (int)sizeof(T) + 7) / 8;
  static_assert(kWords >= kTile * kCt, "the factors fit the staging area");
  __shared__ __attribute__((aligned(16))) double smem_raw[kWords];   // 16-byte LDS reads of K
  T* smem = reinterpret_cast<T*>(smem_raw);
  T* As = smem;
  T* Bs = smem + kTile * kLd;
  T* S = smem;
  __bf16* Ks = reinterpret_cast<__bf16*>(smem_raw);
  double* fac = smem_raw;
  __shared__ double lse[kTile];
  // (the float64 engine keeps its k loop on the run-time head size: unrolled,
  // it spills)
  const int G = sc.G, n = g.nblk, nr = n * G, d = kF32 ? D : g.d;
  const int ntile = (nr + kTile - 1) / kTile, nb = kTile / G;
  const int r0 = blockIdx.x * kTile;
  const long long bh = bh0 + (long long)blockIdx.y;
  const double* qh = qr + bh * (long long)nr * d;
  const double* kh = kr + bh * (long long)nr * d;
  const long long wt = (long long)blockIdx.y * ntile + blockIdx.x;   // this row tile's scratch
  T* ew = esum + wt * ntile * (long long)(kTile * nb);
  T* mw = emax + wt * ntile * (long long)kTile;
  const int row = threadIdx.x >> 2, part = threadIdx.x & 3;   // 4 threads per tile row
  u32x4 aq[3][kF32 ? D / 32 : 1];
  u32x4 kv[kF32 ? 3 * D / 32 : 1];
  const u32x4* kth = kt + (long long)blockIdx.y * ntile * 3 * (D / 8) * kTile;
  if constexpr (kF32) {
    load_q_operands<D>(qh, nr, r0, scale, aq);
    load_k_share<D>(kth, 0, kv);
  }

  // sweep: per column tile, the row maxima, then every (row, key block) sum
  // relative to them; the running row sum l is rescaled when the maximum grows
  T m = -INFINITY;
  double l = 0.0;
  for (int t = 0; t < ntile; ++t) {
    const int c0 = t * kTile;
    if constexpr (kF32) {
      store_k_share<D>(kv, Ks);
      __syncthreads();
      load_k_share<D>(kth, min(t + 1, ntile - 1), kv);   // (the last tile reloads itself)
      score_tile_f32<D>(aq, Ks, reinterpret_cast<float*>(S));
    } else {
      score_tile(qh, kh, nr, d, r0, c0, scale, As, Bs, S);
    }
    // this thread's 16 columns of its row, the present ones among them, and
    // the row maximum over the present columns of the tile
    const unsigned pb = (unsigned)(pmask[t] >> (part * 16)) & 0xffffu;
    T v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = S[row * kSP + part * 16 + e];
    T tm = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if ((pb >> e) & 1u) tm = larger(tm, v[e]);
    tm = larger(tm, __shfl_xor(tm, 1, kWave));
    tm = larger(tm, __shfl_xor(tm, 2, kWave));
    if (tm > m) {
      if (m > -INFINITY) l *= exp((double)m - (double)tm);
      m = tm;
    }
    // exponentials relative to the running maximum (pad sub-cubes: 0; a row
    // with no present key so far has none in this tile either)
    T rs = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      v[e] = ((pb >> e) & 1u) ? exp_of(v[e] - m) : (T)0;
      rs += v[e];
    }
    // per key block sums: 16 / G whole blocks of this thread (G <= 16), or
    // one block over 2 or 4 threads of the row
    T* et = ew + (long long)t * (kTile * nb) + row * nb;
    switch (G) {
      case 1: fold_blocks<1>(v, et + part * 16); break;
      case 2: fold_blocks<2>(v, et + part * 8); break;
      case 4: fold_blocks<4>(v, et + part * 4); break;
      case 8: fold_blocks<8>(v, et + part * 2); break;
      case 16: fold_blocks<16>(v, et + part); break;
      default: {
        T e = rs + __shfl_xor(rs, 1, kWave);
        if (G == 32) {
          if ((part & 1) == 0) et[part >> 1] = e;
        } else {
          e += __shfl_xor(e, 2, kWave);
          if (part == 0) et[0] = e;
        }
      }
    }
    if (part == 0) mw[(long long)t * kTile + row] = m;
    double ds = (double)rs;
    ds += __shfl_xor(ds, 1, kWave);
    ds += __shfl_xor(ds, 2, kWave);
    l += ds;
    __syncthreads();   // S (and the staged K) are rewritten by the next tile
  }
  if (part == 0) lse[row] = (double)m + log(l);
  __syncthreads();

  // aggregation: P_r[i][j] = mean over the present query sub-cubes a of
  // exp(m_t(a) - lse(a)) * E[a][j]
  const int i0 = r0 / G;
  const unsigned long long qpm = pmask[blockIdx.x];   // present query sub-cubes of the tile
  for (int t0 = 0; t0 < ntile; t0 += kCt) {
    const int ct = min(kCt, ntile - t0);
    for (int u = threadIdx.x; u < kTile * ct; u += kThreads) {
      const int rr = u / ct, tt = u - rr * ct;
      const T mr = mw[(long long)(t0 + tt) * kTile + rr];
      fac[rr * kCt + tt] = mr > -INFINITY ? exp((double)mr - lse[rr]) : 0.0;
    }
    __syncthreads();
    const int j0 = t0 * nb, nj = min(n, (t0 + ct) * nb) - j0;
    for (int u = threadIdx.x; u < nb * nj; u += kThreads) {
      const int bi = u / nj, jj = u - bi * nj;
      const int i = i0 + bi;
      if (i >= n) continue;
      const int tt = jj / nb, bj = jj - tt * nb;
      const T* et = ew + (long long)(t0 + tt) * (kTile * nb) + bj;
      double acc = 0.0;
      int na = 0;
      for (int a = 0; a < G; ++a) {
        const int rr = bi * G + a;
        if (!((qpm >> rr) & 1ull)) continue;
        ++na;
        acc += fac[rr * kCt + tt] * (double)et[rr * nb];
      }
      scores[(bh * n + i) * (long long)n + j0 + jj] = (T)log(acc / (double)na);
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

namespace {

template <typename T>
hipError_t router_t(const double* qr, const double* kr, T* scores, double scale, const Geom& g, int rt, int rh,
                    int rw, hipStream_t s) {
  const SubCube sc = make_subcube(g, rt, rh, rw);
  const long long nr = (long long)g.nblk * sc.G;
  dim3 grid((unsigned)((nr + kTile - 1) / kTile), g.batch * g.heads);
  router_kernel<T><<<grid, kThreads, 0, s>>>(qr, kr, scores, scale, g, sc);
  return hipGetLastError();
}

// Scratch of the one-pass kernel for one (batch*head), in elements of T: the
// sums E and, after them, the running maxima; the float32 kernel also takes
// K's three bf16 terms (kt, 3 * ntile * 64 * d bf16).
size_t onepass_head_elems(const Geom& g, const SubCube& sc, size_t& emax_off) {
  const size_t ntile = ((size_t)g.nblk * sc.G + kTile - 1) / kTile;
  emax_off = ntile * ntile * kTile * (size_t)(kTile / sc.G);
  return emax_off + ntile * ntile * kTile;
}

size_t onepass_head_bytes(const Geom& g, const SubCube& sc, size_t elem) {
  size_t emax_off;
  const size_t ntile = ((size_t)g.nblk * sc.G + kTile - 1) / kTile;
  const size_t kt = elem == 4 ? 3 * ntile * kTile * (size_t)g.d * 2 : 0;
  // three 256-byte alignments, and the presence words (counted per head for
  // simplicity: one copy serves a chunk)
  return onepass_head_elems(g, sc, emax_off) * elem + kt + ntile * 8 + 768;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <typename T>
hipError_t router_onepass_t(const double* qr, const double* kr, T* scores, double scale, const Geom& g, int rt,
                            int rh, int rw, void* workspace, size_t ws_bytes, hipStream_t s) {
  const SubCube sc = make_subcube(g, rt, rh, rw);
  size_t emax_off;
  const size_t e_and_m = onepass_head_elems(g, sc, emax_off);
  const size_t per_head = onepass_head_bytes(g, sc, sizeof(T));
  const int bh_total = g.batch * g.heads;
  const int chunk = (int)std::min<size_t>((size_t)bh_total, ws_bytes / per_head);
  if (chunk < 1) return hipErrorInvalidValue;   // the caller checks the size first
  const long long nr = (long long)g.nblk * sc.G;
  const unsigned ntile = (unsigned)((nr + kTile - 1) / kTile);
  for (int bh0 = 0; bh0 < bh_total; bh0 += chunk) {
    const int hc = std::min(chunk, bh_total - bh0);
    // [E of the chunk][pad][maxima][pad][K's bf16 terms][pad][presence words]
    char* base = static_cast<char*>(workspace);
    T* esum = reinterpret_cast<T*>(base);
    const size_t emax_at = align256((size_t)hc * emax_off * sizeof(T));
    T* emax = reinterpret_cast<T*>(base + emax_at);
    const size_t kt_at = align256(emax_at + (size_t)hc * (e_and_m - emax_off) * sizeof(T));
    u32x4* kt = reinterpret_cast<u32x4*>(base + kt_at);
    const size_t kt_bytes = std::is_same<T, float>::value ? (size_t)hc * 3 * ntile * kTile * g.d * 2 : 0;
    unsigned long long* pmask = reinterpret_cast<unsigned long long*>(base + align256(kt_at + kt_bytes));
    router_present_kernel<<<ntile * kTile / kThreads + 1, kThreads, 0, s>>>(pmask, g, sc, (int)nr);
    if (std::is_same<T, float>::value) {
      const long long items = (long long)ntile * kTile * g.d / 8;
      router_k32_kernel<<<dim3((unsigned)((items + kThreads - 1) / kThreads), hc), kThreads, 0, s>>>(
          kr, kt, (int)nr, g.d, (int)ntile, bh0);
    }
    if (g.d == 64)
      router_onepass_kernel<T, 64><<<dim3(ntile, hc), kThreads, 0, s>>>(qr, kr, scores, esum, emax, kt, pmask,
                                                                        scale, g, sc, bh0);
    else
      router_onepass_kernel<T, 128><<<dim3(ntile, hc), kThreads, 0, s>>>(qr, kr, scores, esum, emax, kt, pmask,
                                                                         scale, g, sc, bh0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t router_workspace_bytes(const Geom& g, int rt, int rh, int rw, size_t elem, int heads) {
  return (size_t)heads * onepass_head_bytes(g, make_subcube(g, rt, rh, rw), elem);
}

namespace {

template <typename T>
hipError_t router_any(const double* qr, const double* kr, T* scores, double scale, const Geom& g, int rt, int rh,
                      int rw, void* workspace, size_t ws_bytes, hipStream_t s) {
  if (workspace == nullptr) return router_t(qr, kr, scores, scale, g, rt, rh, rw, s);
  return router_onepass_t(qr, kr, scores, scale, g, rt, rh, rw, workspace, ws_bytes, s);
}

}  // namespace

hipError_t launch_router(const double* qr, const double* kr, double* scores, double scale, const Geom& g,
                         int rt, int rh, int rw, hipStream_t s, void* workspace, size_t ws_bytes) {
  return router_any(qr, kr, scores, scale, g, rt, rh, rw, workspace, ws_bytes, s);
}

hipError_t launch_router(const double* qr, const double* kr, float* scores, double scale, const Geom& g,
                         int rt, int rh, int rw, hipStream_t s, void* workspace, size_t ws_bytes) {
  return router_any(qr, kr, scores, scale, g, rt, rh, rw, workspace, ws_bytes, s);
}

}  // namespace sa
