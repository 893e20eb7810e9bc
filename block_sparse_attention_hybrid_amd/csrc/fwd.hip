// Block-sparse attention forward over per-row kept-block lists (gfx950).
//
// SpargeAttention2 summary page, "Kernel Implementation of the Hybrid-Masked
// Block-Sparse Attention" (Algorithm 1): for one query block, loop over the
// kept key/value blocks only; per block S = Q K^T * scale, an online softmax
// (running max and running sum, rescaling the output accumulator), O += P V;
// divide by the final sum at the end.  VSA summary page, "The Fine Stage":
// the kernel takes the block-index list directly.  Keys in pad slots of a
// partial cube are masked out (VSA2 section 2.2, "Kernel Implementation").
//
// Mapping to CDNA4.  One workgroup = one query block of 64 tokens = 2 waves
// of 32 queries.  Both products use v_mfma_f32_32x32x16_bf16 in transposed
// form so that the probabilities never leave registers:
//   S^T (32 keys x 32 queries) = K (A operand, rows from LDS) x Q^T (B
//        operand, held in registers for the whole row);
//   O^T (32 dims x 32 queries) += V^T (A operand, from a transposed LDS copy)
//        x P^T (B operand).
// The accumulator layout of the first product gives every lane one query and
// 16 of its keys per 32-key tile; the second product's B operand wants one
// query and 8 keys per lane, which is a subset of the same registers once
// its k index is permuted -- and V^T's LDS reads use the same permutation.
// Row statistics (max, sum) therefore live per lane; the two half-waves that
// share a query combine their maxima with one cross-lane exchange.
//
// K and V tiles (16 KB each at d = 128) are staged through LDS and shared by
// the two waves; the next kept block's tiles are fetched into registers while
// the current one is computed.  Rows are mapped to workgroups so that each
// XCD (workgroups are dispatched round-robin over the 8 XCDs) processes a
// contiguous range of rows: neighbouring query blocks of a head, whose kept
// lists overlap, then share K/V tiles in that XCD's L2.
#include "sa_launch.h"

#include <math.h>

namespace sa {

namespace {

constexpr int kThreads = 128;
constexpr int kXcds = 8;
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

template <int D>
struct Tile {
  static constexpr int kLdK = D + 8;     // bf16 per K row in LDS (16-byte pad)
  static constexpr int kLdV = 64 + 4;    // bf16 per V^T row in LDS (8-byte pad)
  static constexpr int kCpr = D / 8;     // 16-byte chunks per K/V row
  static constexpr int kKLoads = 64 * kCpr / kThreads;        // K chunks per thread
  static constexpr int kVTiles = (64 / 4) * kCpr / kThreads;  // 4x8 V micro-tiles per thread
};

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_kernel(const bf16* __restrict__ qc,
                                                       const bf16* __restrict__ kc,
                                                       const bf16* __restrict__ vc,
                                                       const int32_t* __restrict__ lut,
                                                       const int32_t* __restrict__ counts, int cap,
                                                       Geom g, float sc_log2, bf16* __restrict__ oc,
                                                       float* __restrict__ lse_c, int rows,
                                                       int per_xcd) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) bf16 Ks[64 * T::kLdK];
  __shared__ __attribute__((aligned(16))) bf16 Vt[D * T::kLdV];

  const int w = blockIdx.x;
  const int row = (w % kXcds) * per_xcd + w / kXcds;
  if (row >= rows) return;
  const long long bh = row / g.nblk;
  const int i = row - (int)(bh * g.nblk);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, ql = lane & 31;
  const int q = wave * 32 + ql;  // query slot in the block

  const long long head_off = bh * g.n_pad * D;
  const bf16* kh = kc + head_off;
  const bf16* vh = vc + head_off;

  // Q^T operand: this lane's query, dims 16*ds + 8*h .. +7
  bf16x8 qreg[D / 16];
  {
    const u32x4* qrow = reinterpret_cast<const u32x4*>(qc + head_off + ((long long)i * 64 + q) * D);
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) qreg[ds] = as_bf16x8(qrow[2 * ds + h]);
  }

  int count = counts[row];
  count = count < 0 ? 0 : (count > cap ? cap : count);
  const int32_t* lrow = lut + (long long)row * cap;

  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  float m = -INFINITY, l = 0.f;

  // register staging of one K/V tile
  u32x4 kreg[T::kKLoads];
  u32x4 vreg[T::kVTiles][4];
  auto load_tile = [&](int j) {
    const u32x4* kb = reinterpret_cast<const u32x4*>(kh + (long long)j * 64 * D);
    const u32x4* vb = reinterpret_cast<const u32x4*>(vh + (long long)j * 64 * D);
#pragma unroll
    for (int r = 0; r < T::kKLoads; ++r) kreg[r] = kb[tid + kThreads * r];
#pragma unroll
    for (int r = 0; r < T::kVTiles; ++r) {
      const int mt = tid + kThreads * r;
      const int kg = mt % 16, dc = mt / 16;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) vreg[r][kk] = vb[(4 * kg + kk) * T::kCpr + dc];
    }
  };
  auto store_tile = [&](uint64_t real) {
#pragma unroll
    for (int r = 0; r < T::kKLoads; ++r) {
      const int c = tid + kThreads * r;
      const int key = c / T::kCpr, ch = c % T::kCpr;
      u32x4 v = kreg[r];
      if (!((real >> key) & 1ull)) v = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&Ks[key * T::kLdK + ch * 8]) = v;
    }
#pragma unroll
    for (int r = 0; r < T::kVTiles; ++r) {
      const int mt = tid + kThreads * r;
      const int kg = mt % 16, dc = mt / 16;
      u32x4 x[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        x[kk] = ((real >> (4 * kg + kk)) & 1ull) ? vreg[r][kk] : u32x4{0u, 0u, 0u, 0u};
      // transpose a 4 (keys) x 8 (dims) micro-tile into 8 rows of 4 keys
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int word = dd >> 1, hi = dd & 1;
        uint32_t e[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) e[kk] = hi ? (x[kk][word] >> 16) : (x[kk][word] & 0xffffu);
        u32x2 pk = {e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
        *reinterpret_cast<u32x2*>(&Vt[(8 * dc + dd) * T::kLdV + 4 * kg]) = pk;
      }
    }
  };
  auto lut_at = [&](int it, bool& ok) -> int {
    const int j = lrow[it];
    ok = (j >= 0 && j < g.nblk);
    return ok ? j : 0;
  };

  bool ok_cur = false;
  int j_cur = 0;
  if (count > 0) {
    j_cur = lut_at(0, ok_cur);
    load_tile(j_cur);
    store_tile(ok_cur ? block_real_mask(g, j_cur) : 0ull);
  }
  for (int it = 0; it < count; ++it) {
    const uint64_t real = ok_cur ? block_real_mask(g, j_cur) : 0ull;
    bool ok_next = false;
    int j_next = 0;
    __syncthreads();
    if (it + 1 < count) {
      j_next = lut_at(it + 1, ok_next);
      load_tile(j_next);
    }

    // S^T = K Q^T for keys 0..31 and 32..63
    f32x16 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[kt][r] = 0.f;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[(32 * kt + ql) * T::kLdK + 16 * ds + 8 * h]);
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ds], st[kt], 0, 0, 0);
      }
    }
    // scale into the log2 domain, mask pad keys, row max
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kt + 8 * (r >> 2) + 4 * h + (r & 3);
        float v = st[kt][r] * sc_log2;
        if (!((real >> key) & 1ull)) v = -INFINITY;
        st[kt][r] = v;
        mloc = fmaxf(mloc, v);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m, mloc);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    float lsum = 0.f;
    uint32_t pw[2][8];  // P^T as packed bf16 pairs, in register order
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(st[kt][r] - m_use);
        const float p1 = __builtin_amdgcn_exp2f(st[kt][r + 1] - m_use);
        lsum += p0 + p1;
        pw[kt][r >> 1] = pack_bf16x2(p0, p1);
      }
    l = l * alpha + lsum;
    m = m_new;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;

    // O^T += V^T P^T; k-step ks covers registers 8*(ks%2) .. +7 of key tile ks/2
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kt = ks >> 1, a0 = 2 * (ks & 1);
      const u32x4 bw = {pw[kt][4 * (ks & 1)], pw[kt][4 * (ks & 1) + 1], pw[kt][4 * (ks & 1) + 2],
                        pw[kt][4 * (ks & 1) + 3]};
      const bf16x8 b = as_bf16x8(bw);
      const int key0 = 32 * kt + 8 * a0 + 4 * h;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const bf16* vrow = &Vt[(32 * dt + ql) * T::kLdV];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + key0);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + key0 + 8);
        const u32x4 aw = {lo[0], lo[1], hi[0], hi[1]};
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aw), b, acc[dt], 0, 0, 0);
      }
    }
    __syncthreads();
    if (it + 1 < count) store_tile(ok_next ? block_real_mask(g, j_next) : 0ull);
    j_cur = j_next;
    ok_cur = ok_next;
  }

  // epilogue: O = acc / l, LSE = (m + log2 l) ln 2; pad queries and empty rows -> 0, -inf
  const float l_tot = l + __shfl_xor(l, 32, 64);
  const bool qreal = (block_real_mask(g, i) >> q) & 1ull;
  const bool live = qreal && l_tot > 0.f;
  const float inv = live ? 1.f / l_tot : 0.f;
  bf16* orow = oc + head_off + ((long long)i * 64 + q) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const u32x2 v = {pack_bf16x2(acc[dt][4 * a] * inv, acc[dt][4 * a + 1] * inv),
                       pack_bf16x2(acc[dt][4 * a + 2] * inv, acc[dt][4 * a + 3] * inv)};
      *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * a + 4 * h) = v;
    }
  if (h == 0) {
    lse_c[bh * g.n_pad + (long long)i * 64 + q] = live ? (m + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

size_t fwd_workspace_bytes(const Geom&) { return 0; }

hipError_t launch_fwd(const void* qc, const void* kc, const void* vc, const int32_t* lut,
                      const int32_t* counts, int cap, const Geom& g, float scale, void* oc,
                      float* lse_c, void*, hipStream_t s) {
  const long long rows = (long long)g.batch * g.heads * g.nblk;
  const int per_xcd = (int)((rows + kXcds - 1) / kXcds);
  const float sc_log2 = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)(per_xcd * kXcds));
  if (g.d == 128) {
    fwd_kernel<128><<<grid, kThreads, 0, s>>>(static_cast<const bf16*>(qc), static_cast<const bf16*>(kc),
                                              static_cast<const bf16*>(vc), lut, counts, cap, g, sc_log2,
                                              static_cast<bf16*>(oc), lse_c, (int)rows, per_xcd);
  } else {
    fwd_kernel<64><<<grid, kThreads, 0, s>>>(static_cast<const bf16*>(qc), static_cast<const bf16*>(kc),
                                             static_cast<const bf16*>(vc), lut, counts, cap, g, sc_log2,
                                             static_cast<bf16*>(oc), lse_c, (int)rows, per_xcd);
  }
  return hipGetLastError();
}

}  // namespace sa
