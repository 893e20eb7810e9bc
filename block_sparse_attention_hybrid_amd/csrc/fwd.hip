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
// Mapping to CDNA4.  One wavefront owns one query block (64 queries) for the
// whole row, so every K/V byte brought into the CU is used by all 64 queries.
// Both products run on v_mfma_f32_32x32x16_bf16 in transposed form:
//   S^T (32 keys x 32 queries) = K (A operand) x Q^T (B operand),
//   O^T (32 dims x 32 queries) += V^T (A operand) x P^T (B operand).
// The accumulator layout of the first product leaves every lane with one
// query and 16 of its keys per 32-key tile.  The K rows fed to lane r are
// permuted (sigma below) so that, for each 16-key step of the second product,
// a lane's 8 probabilities belong to 8 consecutive keys -- exactly the 8 keys
// the V layout stores in that lane's 16-byte chunk.  P therefore never leaves
// registers, and every K and V operand is one fully coalesced 1 KB wave load
// (the QK and V block layouts of sa_layout.h).  The 16 KB of Q operands sit in
// LDS for the whole row.
//
// Software pipeline: the next block's K tile is requested as soon as the
// current S^T is computed and its V tile as soon as the current O update is
// issued, so each load has a GEMM plus a softmax of lead time.  The running
// max is only raised when a block's max exceeds it by more than 2^8 (in the
// base-2 exponent), which leaves the result exact (the final O/l ratio does
// not depend on the reference max) and skips almost every rescale of the
// 128-register output accumulator.
#include "sa_launch.h"

#include <math.h>

namespace sa {

namespace {

constexpr int kXcds = 8;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kStaleMax = 8.f;  // allowed growth of the base-2 exponent before a rescale

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <int D>
__global__ __launch_bounds__(64) void fwd_kernel(const u32x4* __restrict__ qc,
                                                 const u32x4* __restrict__ kc,
                                                 const u32x4* __restrict__ vc,
                                                 const int32_t* __restrict__ lut,
                                                 const int32_t* __restrict__ counts, int cap, Geom g,
                                                 float sc_log2, bf16* __restrict__ oc,
                                                 float* __restrict__ lse_c, int rows, int per_xcd) {
  constexpr int NDS = D / 16;     // 16-dim steps of S^T
  constexpr int NDT = D / 32;     // 32-dim tiles of O^T
  constexpr int BLK = 64 * D / 8; // 16-byte units per block

  // workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous run of rows so neighbouring query blocks (overlapping lists)
  // share K/V tiles in that XCD's L2
  const int w = blockIdx.x;
  const int row = (w % kXcds) * per_xcd + w / kXcds;
  if (row >= rows) return;
  const long long bh = row / g.nblk;
  const int i = row - (int)(bh * g.nblk);

  const int lane = threadIdx.x;
  const int hf = lane >> 5, r = lane & 31;
  // K row fed to A-operand lane r: sigma(8a + 4b + c) = 16(a/2) + 8b + 4(a%2) + c
  const int sig = 16 * (r >> 4) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
  const int kpos = hf * 32 + sig;

  const long long head = bh * (g.n_pad / 64) * (long long)BLK;
  const u32x4* qb = qc + head + (long long)i * BLK;
  const u32x4* kh = kc + head;
  const u32x4* vh = vc + head;

  // Q^T operand chunks live in LDS (each lane reads back its own 16 bytes, so
  // the reads are conflict-free); registers are kept for K, V, S, P and O
  __shared__ u32x4 qlds[2 * NDS * 64];
#pragma unroll
  for (int c = 0; c < 2 * NDS; ++c) qlds[c * 64 + lane] = qb[c * 64 + lane];
  __syncthreads();

  int count = counts[row];
  count = count < 0 ? 0 : (count > cap ? cap : count);
  const int32_t* lrow = lut + (long long)row * cap;

  f32x16 acc[NDT][2];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][qt][e] = 0.f;
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

  u32x4 kreg[2][NDS];
  u32x4 vreg[NDT][4];
  auto valid_id = [&](int j) { return j >= 0 && j < g.nblk; };
  // bit s set iff slot s of block j holds a real token (one slot per lane)
  auto real_mask = [&](int j) -> uint64_t { return ballot(valid_id(j) && slot_token(g, j, lane) >= 0); };
  auto load_k = [&](int j) {
    const u32x4* kb = kh + (long long)(valid_id(j) ? j : 0) * BLK;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) kreg[kt][ds] = kb[(kt * NDS + ds) * 64 + kpos];
  };
  auto load_v = [&](int j) {
    const u32x4* vb = vh + (long long)(valid_id(j) ? j : 0) * BLK;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) vreg[dt][ks] = vb[(dt * 4 + ks) * 64 + lane];
  };

  int j_cur = count > 0 ? lrow[0] : 0;
  if (count > 0) {
    load_k(j_cur);
    load_v(j_cur);
  }
  for (int it = 0; it < count; ++it) {
    const int j_next = (it + 1 < count) ? lrow[it + 1] : 0;
    const uint64_t real = real_mask(j_cur);
    const bool full = real == ~0ull;   // wave-uniform: most blocks have no pad slot
    // this lane's 32 key bits: byte (kt, g) = keys 32 kt + 16 g + 8 hf .. +7
    const uint32_t lmask = (uint32_t)((real >> (8 * hf)) & 0xffu) |
                           ((uint32_t)((real >> (16 + 8 * hf)) & 0xffu) << 8) |
                           ((uint32_t)((real >> (32 + 8 * hf)) & 0xffu) << 16) |
                           ((uint32_t)((real >> (48 + 8 * hf)) & 0xffu) << 24);

    // the two 32-query halves are processed one after the other: S^T and P of
    // one half are live at a time, and the softmax of one half can overlap
    // the matrix-core work of the other
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      // S^T tiles of this query half (kt: keys 0-31 / 32-63)
      f32x16 st[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) st[kt][e] = 0.f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const u32x4 qv = qlds[(qt * NDS + ds) * 64 + lane];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[kt][ds]), as_bf16x8(qv), st[kt],
                                                           0, 0, 0);
      }
      if (qt == 1 && it + 1 < count) load_k(j_next);
      __builtin_amdgcn_sched_barrier(0);

      // online softmax in the base-2 domain; register e of tile kt holds key
      // 32 kt + 16 (e / 8) + 8 hf + e % 8, i.e. bit 16 kt + e of lmask.  The
      // scale is positive, so the max is taken on the raw scores and the scale
      // folds into the exponent's fma.
      float mx = -INFINITY;
      if (full) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, st[kt][e]);
      } else {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, ((lmask >> (16 * kt + e)) & 1u) ? st[kt][e] : -INFINITY);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sc_log2;
      const bool grow = mx > m[qt] + kStaleMax;
      if (__any(grow)) {
        const float alpha = grow ? __builtin_amdgcn_exp2f(m[qt] - mx) : 1.f;
        l[qt] *= alpha;
#pragma unroll
        for (int t = 0; t < NDT; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[t][qt][e] *= alpha;
      }
      if (grow) m[qt] = mx;
      const float nmu = m[qt] == -INFINITY ? 0.f : -m[qt];
      uint32_t pw[2][8];
      float ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          float p0 = __builtin_amdgcn_exp2f(fmaf(st[kt][e], sc_log2, nmu));
          float p1 = __builtin_amdgcn_exp2f(fmaf(st[kt][e + 1], sc_log2, nmu));
          if (!full) {
            p0 = ((lmask >> (16 * kt + e)) & 1u) ? p0 : 0.f;
            p1 = ((lmask >> (16 * kt + e + 1)) & 1u) ? p1 : 0.f;
          }
          ls += p0 + p1;
          pw[kt][e >> 1] = pack_bf16x2(p0, p1);
        }
      l[qt] += ls;
      __builtin_amdgcn_sched_barrier(0);

      // O^T += V^T P^T; k-step ks covers keys 16 ks .. +15 = registers
      // 8 (ks % 2) .. +7 of tile ks / 2
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kt = ks >> 1, o4 = 4 * (ks & 1);
        const u32x4 bw = {pw[kt][o4], pw[kt][o4 + 1], pw[kt][o4 + 2], pw[kt][o4 + 3]};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          acc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vreg[dt][ks]), as_bf16x8(bw),
                                                                acc[dt][qt], 0, 0, 0);
      }
    }
    if (it + 1 < count) load_v(j_next);
    j_cur = j_next;
  }

  // epilogue: O = acc / l, LSE = (m + log2 l) ln 2; pad queries and empty rows -> 0, -inf
  const uint64_t qreal = real_mask(i);
  bf16* ob = oc + (bh * g.n_pad + (long long)i * 64) * D;
  float* lb = lse_c + bh * g.n_pad + (long long)i * 64;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float lt = l[qt] + __shfl_xor(l[qt], 32, 64);
    const int q = 32 * qt + r;
    const bool live = ((qreal >> q) & 1ull) && lt > 0.f;
    const float inv = live ? 1.f / lt : 0.f;
    bf16* orow = ob + (long long)q * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const u32x2 v = {pack_bf16x2(acc[dt][qt][4 * a] * inv, acc[dt][qt][4 * a + 1] * inv),
                         pack_bf16x2(acc[dt][qt][4 * a + 2] * inv, acc[dt][qt][4 * a + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * a + 4 * hf) = v;
      }
    if (hf == 0) lb[q] = live ? (m[qt] + __log2f(lt)) * kLn2 : -INFINITY;
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
  const u32x4* q = static_cast<const u32x4*>(qc);
  const u32x4* k = static_cast<const u32x4*>(kc);
  const u32x4* v = static_cast<const u32x4*>(vc);
  if (g.d == 128)
    fwd_kernel<128><<<grid, 64, 0, s>>>(q, k, v, lut, counts, cap, g, sc_log2, static_cast<bf16*>(oc), lse_c,
                                        (int)rows, per_xcd);
  else
    fwd_kernel<64><<<grid, 64, 0, s>>>(q, k, v, lut, counts, cap, g, sc_log2, static_cast<bf16*>(oc), lse_c,
                                       (int)rows, per_xcd);
  return hipGetLastError();
}

}  // namespace sa
