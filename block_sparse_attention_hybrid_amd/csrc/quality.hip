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
//     queries, o from the dense run, and optionally Eq. 8's two terms, the
//     dropped term (p (1 - m)) V and the renormalisation term
//     (1 - 1/tau)(p m) V, as L1 norms relative to the same sum |o|;
//   * ideal block scores (VSA2 section 2.2, the MeanPool of the full attention
//     matrix a router approximates): P_ideal[i][j] = the full softmax mass that
//     block i's real queries put on block j's real keys, averaged over those
//     queries, recomputed from the dense run's LSE on the matrix cores;
//   * recall: the share of the c blocks with the largest P_ideal that a kept
//     list of c blocks holds.
#include "sa_launch.h"

#include <math.h>

namespace sa {

namespace {

constexpr int kMaxRecallWords = 4096 / 32;   // bitmap of up to 4096 blocks

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// One wavefront per query block i, over every key block j: S^T = K Q^T on
// v_mfma_f32_32x32x16_bf16 (K rows as the A operand, one 1 KB chunk per load;
// register e of key tile kt holds key 32 kt + 8 (e / 4) + 4 (lane / 32) + e % 4
// for query lane % 32 of query half qt), P = exp2(S scale log2e - LSE log2e)
// with the dense LSE, summed over the real (query, key) pairs.
template <int D>
__global__ __launch_bounds__(64) void ideal_mass_kernel(const u32x4* __restrict__ qc,
                                                        const u32x4* __restrict__ kc,
                                                        const float* __restrict__ lse_d, Geom g,
                                                        float sc_log2, double* __restrict__ mass) {
  constexpr int NDS = D / 16, BLK = 64 * D / 8;
  const int i = blockIdx.x;
  const long long bh = blockIdx.y;
  const int lane = threadIdx.x, hf = lane >> 5, r = lane & 31;
  const long long head = bh * (long long)g.nblk * BLK;
  u32x4 qreg[2 * NDS];
#pragma unroll
  for (int c = 0; c < 2 * NDS; ++c) qreg[c] = qc[head + (long long)i * BLK + c * 64 + lane];
  const uint64_t qreal = block_real_mask(g, i);
  float l2[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int q = 32 * qt + r;
    const float l = lse_d[bh * g.n_pad + (long long)i * kBlock + q];
    // pad slots and queries without any key contribute nothing
    l2[qt] = ((qreal >> q) & 1ull) && l > -INFINITY ? l * 1.4426950408889634f : INFINITY;
  }
  const double inv_r = 1.0 / (double)block_real_count(g, i);
  double* out = mass + (bh * g.nblk + i) * (long long)g.nblk;
  for (int j = 0; j < g.nblk; ++j) {
    const uint64_t kreal = block_real_mask(g, j);
    u32x4 kreg[2][NDS];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) kreg[kt][ds] = kc[head + (long long)j * BLK + (kt * NDS + ds) * 64 + lane];
    float acc = 0.f;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      f32x16 st[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        st[kt] = f32x16{};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
          st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[kt][ds]), as_bf16x8(qreg[qt * NDS + ds]),
                                                           st[kt], 0, 0, 0);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = 32 * kt + 8 * (e >> 2) + 4 * hf + (e & 3);
          const float p = __builtin_amdgcn_exp2f(fmaf(st[kt][e], sc_log2, -l2[qt]));
          acc += ((kreal >> key) & 1ull) ? p : 0.f;
        }
    }
    const double tot = wave_sum((double)acc);
    if (lane == 0) out[j] = tot * inv_r;
  }
}

// Per row: |kept ids & top ids| / count (1 for an empty list), with the top
// list of the same count selected from P_ideal; a bitmap in LDS marks the kept ids.
__global__ __launch_bounds__(64) void recall_kernel(const int32_t* __restrict__ lut,
                                                    const int32_t* __restrict__ counts, int cap,
                                                    const int32_t* __restrict__ top, int n,
                                                    double* __restrict__ recall) {
  __shared__ uint32_t bits[kMaxRecallWords];
  const long long row = blockIdx.x;
  const int lane = threadIdx.x;
  const int words = (n + 31) / 32;
  for (int w = lane; w < words; w += 64) bits[w] = 0u;
  __syncthreads();
  int c = counts[row];
  c = c < 0 ? 0 : (c > cap ? cap : c);
  const int32_t* kl = lut + row * (long long)cap;
  for (int e = lane; e < c; e += 64) {
    const int j = kl[e];
    if (j >= 0 && j < n) atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  const int32_t* tl = top + row * (long long)n;
  int hit = 0;
  for (int e = lane; e < c; e += 64) {
    const int j = tl[e];
    hit += (j >= 0 && j < n) ? (int)((bits[j >> 5] >> (j & 31)) & 1u) : 0;
  }
  hit = wave_sum(hit);
  if (lane == 0) recall[row] = c == 0 ? 1.0 : (double)hit / (double)c;
}

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

// One wavefront per query block, lane = slot.  With TERMS, Eq. 8's two terms
// are summed as well: per query e_drop = o_d - tau o_s (the dense output of
// the dropped keys, (p (1 - m)) V) and e_ren = (tau - 1) o_s (= (1 - 1/tau)
// (p m) V, since (p m) V = tau o_s).
template <bool TERMS>
__global__ __launch_bounds__(64) void mask_error_kernel(const float* __restrict__ lse_s,
                                                        const float* __restrict__ lse_d,
                                                        const bf16* __restrict__ o_s,
                                                        const bf16* __restrict__ o_d, Geom g,
                                                        float* __restrict__ tau, float* __restrict__ rel,
                                                        float* __restrict__ rel_drop, float* __restrict__ rel_ren) {
  const int i = blockIdx.x;
  const long long bh = blockIdx.y;
  const int s = threadIdx.x, d = g.d;
  const long long slot = bh * g.n_pad + (long long)i * kBlock + s;
  const bool real = slot_token(g, i, s) >= 0;
  const float ld = lse_d[slot], ls = lse_s[slot];
  float t = 0.f;
  if (real && ld > -INFINITY) t = ls > -INFINITY ? expf(ls - ld) : 0.f;
  tau[slot] = t;
  double num = 0.0, den = 0.0, nd = 0.0, nr = 0.0;
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
        if (TERMS) {
          const double td = (double)t;
          nd += fabs((double)y0 - td * x0) + fabs((double)y1 - td * x1);
          nr += (1.0 - td) * ((double)fabsf(x0) + (double)fabsf(x1));
        }
      }
    }
  }
  num = wave_sum(num);
  den = wave_sum(den);
  if (TERMS) {
    nd = wave_sum(nd);
    nr = wave_sum(nr);
  }
  if (s == 0) {
    rel[bh * g.nblk + i] = den > 0.0 ? (float)(num / den) : 0.f;
    if (TERMS) {
      rel_drop[bh * g.nblk + i] = den > 0.0 ? (float)(nd / den) : 0.f;
      rel_ren[bh * g.nblk + i] = den > 0.0 ? (float)(nr / den) : 0.f;
    }
  }
}

}  // namespace

hipError_t launch_pooled_mass(const double* scores, const int32_t* lut, const int32_t* counts, int cap,
                              const Geom& g, double* mass, hipStream_t s) {
  const long long rows = (long long)g.batch * g.heads * g.nblk;
  pooled_mass_kernel<<<(unsigned)rows, 64, 0, s>>>(scores, lut, counts, cap, g.nblk, mass);
  return hipGetLastError();
}

hipError_t launch_mask_error(const float* lse_s, const float* lse_d, const void* o_s, const void* o_d,
                             const Geom& g, float* tau, float* rel, hipStream_t s, float* rel_drop,
                             float* rel_ren) {
  dim3 grid(g.nblk, g.batch * g.heads);
  const bf16* os = static_cast<const bf16*>(o_s);
  const bf16* od = static_cast<const bf16*>(o_d);
  if (rel_drop != nullptr)
    mask_error_kernel<true><<<grid, 64, 0, s>>>(lse_s, lse_d, os, od, g, tau, rel, rel_drop, rel_ren);
  else
    mask_error_kernel<false><<<grid, 64, 0, s>>>(lse_s, lse_d, os, od, g, tau, rel, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_ideal_mass(const void* qc, const void* kc, const float* lse_d, const Geom& g, float scale,
                             double* mass, hipStream_t s) {
  dim3 grid(g.nblk, g.batch * g.heads);
  const float sc_log2 = scale * 1.4426950408889634f;
  const u32x4* q = static_cast<const u32x4*>(qc);
  const u32x4* k = static_cast<const u32x4*>(kc);
  if (g.d == 128)
    ideal_mass_kernel<128><<<grid, 64, 0, s>>>(q, k, lse_d, g, sc_log2, mass);
  else
    ideal_mass_kernel<64><<<grid, 64, 0, s>>>(q, k, lse_d, g, sc_log2, mass);
  return hipGetLastError();
}

hipError_t launch_recall(const int32_t* lut, const int32_t* counts, int cap, const int32_t* top, const Geom& g,
                         double* recall, hipStream_t s) {
  const long long rows = (long long)g.batch * g.heads * g.nblk;
  recall_kernel<<<(unsigned)rows, 64, 0, s>>>(lut, counts, cap, top, g.nblk, recall);
  return hipGetLastError();
}

}  // namespace sa
