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
// (the QK and V block layouts of sa_layout.h).  The 16 KB of Q operands stay
// in registers for the whole row, so the loop touches no LDS at all.
//
// Software pipeline: the next block's K tile is requested as soon as the
// current S^T is computed and its V tile as soon as the current O update is
// issued, so each load has a GEMM plus a softmax of lead time.
//
// Online softmax without a per-block row max: the exponentials of a block are
// taken against the running reference m at once, and only when a lane's sum
// over its 32 probabilities of a half exceeds 2^8 (so some probability could
// be large) or m is still unset is the exact block max taken, m raised, the
// accumulator rescaled and the probabilities redone.  The final O / l does
// not depend on m, so the result is the same; every probability that reaches
// the products is at most 2^8, and the rare slow path replaces a max over 64
// scores per block.
#include "sa_launch.h"
#include "sa_rowmap.h"

#include <math.h>

#include <type_traits>

namespace sa {

namespace {

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kSumLimit = 256.f;  // a lane's block sum above this triggers an exact-max rescale

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Division by a run-time constant d (1 <= d < 2^24) for n < 2^24 with one
// high multiply, an add and a shift (round-up multiplier method).
struct FastDiv {
  uint32_t m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1u << l) < d) ++l;
  FastDiv f;
  f.m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
  f.l = l;
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) { return (__umulhi(n, f.m) + n) >> f.l; }

// block index -> cube coordinates: divisions by nw and nh
struct CubeDiv {
  FastDiv w, h;
};

// Start value of a score accumulator: -inf for a pad key (bit b of pad set),
// 0 otherwise.  The sign-extended one-bit field is all ones or zero, and its
// AND with the bits of -inf gives -inf or +0: two plain VALU operations (the
// opaque copy keeps the compiler from turning them back into a compare and a
// select, which costs a VCC hazard wait per element).
__device__ __forceinline__ float pad_start(uint32_t pad, int b) {
  int t = __builtin_amdgcn_sbfe((int)pad, b, 1);
  asm volatile("" : "+v"(t));
  return __uint_as_float((uint32_t)t & 0xff800000u);
}

// Groups of neighbouring query blocks that fwd_group_kernel (below) runs with
// K/V shared through LDS when their lists are dense.
#ifndef SA_FWD_DENSE_DIV
#define SA_FWD_DENSE_DIV 4
#endif
constexpr int kDenseDiv = SA_FWD_DENSE_DIV;   // dense: mean list >= nblk / kDenseDiv (0: never)
#ifndef SA_FWD_DENSE_HEAD_MB
#define SA_FWD_DENSE_HEAD_MB 32
#endif
constexpr size_t kDenseHeadBytes = (size_t)SA_FWD_DENSE_HEAD_MB << 20;   // K/V bytes per head
constexpr int kGroup = 4;     // waves (query blocks) per workgroup
constexpr int kSlots = 4;     // LDS ring of K/V tiles
constexpr int kMaxBlocks = 4096;

// Whether the group of query block i (blocks 4 (i/4) .. +3 of head bh) is dense.
__device__ __forceinline__ bool group_dense(const int32_t* __restrict__ counts, int cap, int nblk, long long bh,
                                            int i, int dense_div) {
  const int i0 = i & ~(kGroup - 1);
  const int active = min(kGroup, nblk - i0);
  long long sum = 0;
  for (int w = 0; w < active; ++w) {
    int c = counts[bh * nblk + i0 + w];
    sum += c < 0 ? 0 : (c > cap ? cap : c);
  }
  return sum * dense_div >= (long long)active * nblk;
}

// The state of one wavefront's query block (64 queries, two 32-query halves)
// and the steps of one kept key block, shared by both forward kernels: Q^T
// operands, the O^T accumulators, the running reference m and sum l per
// half, and the K and V operands of the current block (filled by the caller,
// from global memory or from LDS).
template <int D>
struct RowState {
  static constexpr int NDS = D / 16;       // 16-dim steps of S^T
  static constexpr int NDT = D / 32;       // 32-dim tiles of O^T
  static constexpr int G1 = 2 * NDS;       // MFMA steps of S^T for one half
  static constexpr int G2 = 4 * NDT;       // MFMA steps of O^T for one half

  u32x4 qreg[2 * NDS];      // Q^T operand chunks, in registers for the whole row
  u32x4 kreg[2][NDS];       // K operands of the current block: [32-key tile][dim step]
  u32x4 vreg[NDT][4];       // V operands: [32-dim tile][16-key step]
  f32x16 acc[NDT][2];
  float m[2], l[2];
  float sc_log2;
  int hf;                   // lane / 32
  int lt, lh, lw;           // cube offsets of this lane's slot
  const Geom* g;
  CubeDiv cd;

  __device__ __forceinline__ void init(const Geom& geom, const CubeDiv& div, float scl2, int lane) {
    g = &geom;
    cd = div;
    sc_log2 = scl2;
    hf = lane >> 5;
    slot_offsets(geom, lane, lt, lh, lw);
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][qt][e] = 0.f;
    m[0] = m[1] = -INFINITY;
    l[0] = l[1] = 0.f;
  }

  // bit s set iff slot s of block j holds a real token; the cube coordinates
  // are uniform (scalar unit), only partial cubes need a per-lane test
  __device__ __forceinline__ uint64_t real_mask(int j) const {
    const bool ok = j >= 0 && j < g->nblk;
    const uint32_t jj = ok ? (uint32_t)j : 0u;
    const uint32_t r = fdiv(jj, cd.w);
    const int bw = (int)jj - (int)r * g->nw;
    const int bt = (int)fdiv(r, cd.h);
    const int bhh = (int)r - bt * g->nh;
    const int rt = min(g->ct, g->frames - bt * g->ct);
    const int rh = min(g->ch, g->height - bhh * g->ch);
    const int rw = min(g->cw, g->width - bw * g->cw);
    const uint64_t b = ballot(lt < rt && lh < rh && lw < rw);
    return ok ? b : 0ull;
  }

  // this lane's 32 key bits: byte (kt, g) = keys 32 kt + 16 g + 8 hf .. +7
  __device__ __forceinline__ uint32_t lane_mask(uint64_t real) const {
    return (uint32_t)((real >> (8 * hf)) & 0xffu) | ((uint32_t)((real >> (16 + 8 * hf)) & 0xffu) << 8) |
           ((uint32_t)((real >> (32 + 8 * hf)) & 0xffu) << 16) |
           ((uint32_t)((real >> (48 + 8 * hf)) & 0xffu) << 24);
  }

  __device__ __forceinline__ u32x4 qchunk(int qt, int ds) const { return qreg[qt * NDS + ds]; }

  // S^T = K Q^T, one MFMA per step (16 steps: ds = step / 2, kt = step % 2);
  // q holds the Q^T chunk of this step's ds
  __device__ __forceinline__ void gemm1_step(f32x16 (&st)[2], const u32x4& q, int step) {
    const int ds = step >> 1, kt = step & 1;
    st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[kt][ds]), as_bf16x8(q), st[kt], 0, 0, 0);
  }

  // Register e of tile kt holds key 32 kt + 16 (e / 8) + 8 hf + e % 8, i.e.
  // bit 16 kt + e of the lane's key mask.  Pad keys of a partial block get
  // S = -inf (so P = 0 and they never set the max) by starting their
  // accumulators at -inf instead of 0: the first MFMA of each tile reads the
  // start value, so a full block (wave-uniform branch) keeps the free zero
  // operand and a partial one pays two plain operations per start value.
  __device__ __forceinline__ void gemm1_first(f32x16 (&st)[2], const u32x4& q, uint64_t real) {
    if (real == ~0ull) {
      const f32x16 z = {};
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[kt][0]), as_bf16x8(q), z, 0, 0, 0);
    } else {
      const uint32_t pad = ~lane_mask(real);   // bit set: pad key
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x16 init;
#pragma unroll
        for (int e = 0; e < 16; ++e) init[e] = pad_start(pad, 16 * kt + e);
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[kt][0]), as_bf16x8(q), init, 0, 0, 0);
      }
    }
  }

  // the whole S^T half in one region
  __device__ __forceinline__ void gemm1_half(int qt, f32x16 (&st)[2], uint64_t real) {
    gemm1_first(st, qchunk(qt, 0), real);
#pragma unroll
    for (int k = 2; k < G1; ++k) gemm1_step(st, qchunk(qt, k >> 1), k);
  }

  // one register pair of P = exp2(scale S - m) (bf16-packed) and its sum
  __device__ __forceinline__ void exp_pair(const f32x16 (&st)[2], uint32_t (&pw)[2][8], float nmu, float& ls,
                                           int step) const {
    const int kt = step >> 3, e = 2 * (step & 7);
    const float p0 = __builtin_amdgcn_exp2f(fmaf(st[kt][e], sc_log2, nmu));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(st[kt][e + 1], sc_log2, nmu));
    ls += p0 + p1;
    pw[kt][e >> 1] = pack_bf16x2(p0, p1);
  }

  // row max of one half (raw scores; the scale is positive)
  __device__ __forceinline__ float half_max(const f32x16 (&st)[2]) const {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, st[kt][e]);
    // the two half-waves hold the two halves of every query's keys
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sc_log2;
  }

  // O^T += V^T P^T, one MFMA per step (16 steps: ks = step / NDT, dt =
  // step % NDT at d = 128); k-step ks covers keys 16 ks .. +15 = registers
  // 8 (ks % 2) .. +7 of tile ks / 2
  __device__ __forceinline__ void gemm2_step(int qt, const uint32_t (&pw)[2][8], int step) {
    const int ks = step / NDT, dt = step % NDT;
    const int kt = ks >> 1, o4 = 4 * (ks & 1);
    const u32x4 bw = {pw[kt][o4], pw[kt][o4 + 1], pw[kt][o4 + 2], pw[kt][o4 + 3]};
    acc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vreg[dt][ks]), as_bf16x8(bw), acc[dt][qt],
                                                          0, 0, 0);
  }

  // empty asm "uses": keep a stage's results computed in its own region (the
  // compiler would otherwise sink the softmax past the next branch and lose
  // the overlap with the matrix cores)
  static __device__ __forceinline__ void pin(const uint32_t (&pw)[2][8]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 8; ++e) asm volatile("" ::"v"(pw[kt][e]));
  }

  // The exponentials of a half are computed with the current m right away and
  // checked afterwards through their sum; the rare half whose sum exceeds the
  // limit, or that finds m unset (always the first block), takes the exact
  // max, raises m, rescales the accumulator and is redone with the new m.
  __device__ __forceinline__ void settle(int qt, const f32x16 (&st)[2], uint32_t (&pw)[2][8], float& ls) {
    const bool trig = !(ls <= kSumLimit) || m[qt] == -INFINITY;
    if (__any(trig)) {
      const float mx = half_max(st);
      const float mn = fmaxf(m[qt], mx);
      const float alpha = (m[qt] == -INFINITY || mn == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[qt] - mn);
      m[qt] = mn;
      l[qt] *= alpha;
#pragma unroll
      for (int t = 0; t < NDT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][qt][e] *= alpha;
      const float nmu = m[qt] == -INFINITY ? 0.f : -m[qt];
      ls = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) exp_pair(st, pw, nmu, ls, k);
    }
    l[qt] += ls;
  }

  __device__ __forceinline__ float neg_m(int qt) const { return m[qt] == -INFINITY ? 0.f : -m[qt]; }

  // O = acc / l, LSE = (m + log2 l) ln 2 of query block i of (batch, head) bh;
  // pad queries and empty rows -> 0, -inf.  TOK = false: O and LSE slot-major
  // (oc [.., n_pad, D], lse_c [.., n_pad]); TOK = true: straight to token order
  // (o [.., N, D], lse [.., N]), pad slots not written -- the inverse
  // re-indexing fused into the epilogue.
  template <bool TOK>
  __device__ __forceinline__ void epilogue(long long bh, int i, int r, bf16* __restrict__ oc,
                                           float* __restrict__ lse_c) const {
    const Geom& G = *g;
    const uint64_t qreal = real_mask(i);
    bf16* ob = oc + (bh * G.n_pad + (long long)i * 64) * D;
    float* lb = lse_c + bh * G.n_pad + (long long)i * 64;
    // token order: cube coordinates of this query block (one division each on the scalar unit)
    int ct0 = 0, ch0 = 0, cw0 = 0;
    if (TOK) {
      const uint32_t rr = fdiv((uint32_t)i, cd.w);
      cw0 = (i - (int)rr * G.nw) * G.cw;
      const int bt = (int)fdiv(rr, cd.h);
      ch0 = ((int)rr - bt * G.nh) * G.ch;
      ct0 = bt * G.ct;
    }
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float ltot = l[qt] + __shfl_xor(l[qt], 32, 64);
      const int q = 32 * qt + r;
      const bool real_q = (qreal >> q) & 1ull;
      const bool live = real_q && ltot > 0.f;
      const float inv = live ? 1.f / ltot : 0.f;
      bf16* orow = ob + (long long)q * D;
      long long tok = 0;
      if (TOK) {
        int tt, hh, ww;
        slot_offsets(G, q, tt, hh, ww);
        tok = ((long long)(ct0 + tt) * G.height + (ch0 + hh)) * G.width + (cw0 + ww);
        orow = oc + (bh * G.n_real + tok) * D;
        if (!real_q) continue;   // pad slots have no token row
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const u32x2 v = {pack_bf16x2(acc[dt][qt][4 * a] * inv, acc[dt][qt][4 * a + 1] * inv),
                           pack_bf16x2(acc[dt][qt][4 * a + 2] * inv, acc[dt][qt][4 * a + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * a + 4 * hf) = v;
        }
      const float lse_q = live ? (m[qt] + __log2f(ltot)) * kLn2 : -INFINITY;
      if (hf == 0) {
        if (TOK)
          lse_c[bh * G.n_real + tok] = lse_q;
        else
          lb[q] = lse_q;
      }
    }
  }
};

// One query block (row of batch*heads*nblk) of the forward, by one wavefront,
// with K and V straight from global memory (L2) into registers.
template <int D, bool TOK>
__device__ __forceinline__ void fwd_row(int row, const u32x4* __restrict__ qc, const u32x4* __restrict__ kc,
                                        const u32x4* __restrict__ vc, const int32_t* __restrict__ lut,
                                        const int32_t* __restrict__ counts, int cap, const Geom& g,
                                        float sc_log2, bf16* __restrict__ oc, float* __restrict__ lse_c,
                                        const CubeDiv& cd, int qg_shift, int dense_div = 0) {
  using RS = RowState<D>;
  constexpr int NDS = RS::NDS, NDT = RS::NDT, G1 = RS::G1, G2 = RS::G2;
  constexpr int BLK = 64 * D / 8; // 16-byte units per block

  const long long bh = row / g.nblk;
  const int i = row - (int)(bh * g.nblk);

  const int lane = threadIdx.x & 63;
  const int hf = lane >> 5, r = lane & 31;
  // K row fed to A-operand lane r: sigma(8a + 4b + c) = 16(a/2) + 8b + 4(a%2) + c
  const int sig = 16 * (r >> 4) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
  const int kpos = hf * 32 + sig;

  const long long head = bh * (g.n_pad / 64) * (long long)BLK;
  const u32x4* qb = qc + head + (long long)i * BLK;
  const u32x4* kh = kc + head;
  const u32x4* vh = vc + head;

  RS S;
#pragma unroll
  for (int c = 0; c < 2 * NDS; ++c) S.qreg[c] = qb[c * 64 + lane];

  // the list of this query block: one per cube, or one per group of
  // 2^qg_shift consecutive cubes (asymmetric query blocks)
  const int nlists = (g.nblk + (1 << qg_shift) - 1) >> qg_shift;
  const long long lrow_i = bh * nlists + (i >> qg_shift);
  int count = counts[lrow_i];
  count = count < 0 ? 0 : (count > cap ? cap : count);
  const int32_t* lrow = lut + lrow_i * cap;
  // rows of dense groups are left to fwd_group_kernel (the check's loads are
  // queued behind those of Q, so they add no latency of their own)
  if (dense_div > 0 && group_dense(counts, cap, g.nblk, bh, i, dense_div)) return;

  S.init(g, cd, sc_log2, lane);
  auto valid_id = [&](int j) { return j >= 0 && j < g.nblk; };
  // both tiles are requested in the order the products consume them, so a
  // product waits only for the chunks it uses
  auto load_k = [&](int j) {
    const u32x4* kb = kh + (long long)(valid_id(j) ? j : 0) * BLK;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) S.kreg[kt][ds] = kb[(kt * NDS + ds) * 64 + kpos];
  };
  auto load_v = [&](int j) {
    const u32x4* vb = vh + (long long)(valid_id(j) ? j : 0) * BLK;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) S.vreg[dt][ks] = vb[(dt * 4 + ks) * 64 + lane];
  };

  // Software pipeline over the kept blocks, per block t (halves 0 and 1):
  //   S^T(t,1) with exp(t,0) | settle(t,0) | O += (t,0) with exp(t,1) |
  //   settle(t,1) | O += (t,1) and S^T(t+1,0)
  // The exp steps are written between the MFMA steps and fenced with
  // scheduling barriers, so the vector units work through one half's softmax
  // while the matrix cores run the other half's product.  K(t+1) is requested
  // once S^T(t,1) is issued, V(t+1) once O(t,1) is.
  f32x16 stA[2], stB[2];
  uint32_t pA[2][8], pB[2][8];
  int j_cur = count > 0 ? lrow[0] : 0;
  uint64_t real = 0;
  if (count > 0) {
    load_k(j_cur);
    load_v(j_cur);
    real = S.real_mask(j_cur);
    S.gemm1_half(0, stA, real);
  }
  // the list entry of the next block is read one iteration ahead
  int j_ahead = count > 1 ? lrow[1] : j_cur;
  for (int it = 0; it < count; ++it) {
    // past the last block the "next" block is the current one again: the
    // pipeline then does one redundant S^T half and reload instead of
    // branching, which keeps each stage one straight-line region
    const int j_next = j_ahead;
    j_ahead = lrow[it + 2 < count ? it + 2 : count - 1];
    uint64_t real_next;
    {
      const float nmu = S.neg_m(0);
      float ls = 0.f;
      S.gemm1_first(stB, S.qchunk(1, 0), real);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k + 2 < G1) S.gemm1_step(stB, S.qchunk(1, (k + 2) >> 1), k + 2);
        S.exp_pair(stA, pA, nmu, ls, k);
        __builtin_amdgcn_sched_barrier(0);
      }
      RS::pin(pA);
      load_k(j_next);
      S.settle(0, stA, pA, ls);
    }
    {
      const float nmu = S.neg_m(1);
      float ls = 0.f;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k < G2) S.gemm2_step(0, pA, k);
        S.exp_pair(stB, pB, nmu, ls, k);
        if (k == 4) real_next = S.real_mask(j_next);   // scalar work between matrix ops
        __builtin_amdgcn_sched_barrier(0);
      }
      RS::pin(pB);
      S.settle(1, stB, pB, ls);
    }
#pragma unroll
    for (int k = 0; k < G2; ++k) S.gemm2_step(1, pB, k);
    real = real_next;
    S.gemm1_half(0, stA, real);
    load_v(j_next);
    j_cur = j_next;
  }
  S.template epilogue<TOK>(bh, i, r, oc, lse_c);
}

template <int D, bool TOK>
__global__ __launch_bounds__(64) void fwd_kernel(const u32x4* __restrict__ qc, const u32x4* __restrict__ kc,
                                                 const u32x4* __restrict__ vc, const int32_t* __restrict__ lut,
                                                 const int32_t* __restrict__ counts, int cap, Geom g,
                                                 float sc_log2, bf16* __restrict__ oc, float* __restrict__ lse_c,
                                                 RowMap map, CubeDiv cd, int qg_shift,
                                                 const int32_t* __restrict__ order, int dense_div);

// ---------------------------------------------------------------------------
// Groups of neighbouring query blocks with K/V shared through LDS.
//
// A workgroup of kGroup waves takes kGroup consecutive query blocks of one
// head (wave w: block 4g + w) and walks the union of their kept lists in
// ascending block order.  Each K/V tile of the union is copied once from
// global memory into a ring of kSlots LDS tiles with direct global-to-LDS
// loads (kSlots - 1 tiles in flight ahead of use); every wave whose own list
// holds the block reads its MFMA operands from LDS and runs the same block
// step as fwd_row, in the same (ascending) order, so the result is
// bit-identical to fwd_row's.  The waves pass one barrier per union entry.
//
// Dense lists are where this pays: there the union of four neighbouring
// lists is little longer than one list, and every tile fetched serves up to
// four query blocks.  With sparse lists the union is about twice the summed
// length, so the waves would idle at the barriers; those groups stay with
// fwd_kernel.  A group is dense when its summed count times dense_div is at
// least its number of blocks times nblk.  fwd_kernel skips the rows of dense
// groups and fwd_group_kernel the rows of the others, so every row runs in
// exactly one of the two launches.  A group whose lists are not strictly
// ascending ids in [0, nblk) runs each row with fwd_row instead.

// One 1 KB chunk straight from global memory to LDS, 16 bytes per lane:
// lane l's bytes at gbase + lane16 land at LDS byte address lds + 16 l
// (gbase and lds wave-uniform, lane16 = 16 * lane).  No register receives
// data.  The copy is written out here rather than through the builtin: with
// the builtin the compiler's wait counting makes every LDS read wait for all
// copies in flight, including those of the tiles ahead, which undoes the
// prefetch.  The kernel waits for these copies explicitly instead.  M0 (the
// LDS base of the copy) is a register the compiler reserves, so the block
// saves and restores it itself rather than declaring a clobber, and leaves
// one wait state between setting it and the copy.
__device__ __forceinline__ void chunk_to_lds(uint32_t lds, const void* gbase, uint32_t lane16) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"   // one wait state between writing M0 and the copy that reads it
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(lane16), "s"(gbase)
      : "memory");
#else
  (void)lds;
  (void)gbase;
  (void)lane16;
#endif
}

// s_waitcnt immediate for vmcnt(n) alone (expcnt and lgkmcnt at their maxima)
constexpr int wait_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

template <int D>
struct GroupLds {
  u32x4 ring[kSlots][2 * (64 * D / 8)];
  int32_t ulist[kMaxBlocks];              // union entry: id | member mask << 16
  uint32_t bits[kGroup][kMaxBlocks / 32];
  int wpre[kMaxBlocks / 32 + 1];
  int flag_bad;
};

// One group (row grow of the group map); returns at once unless it is dense.
template <int D, bool TOK>
__device__ __forceinline__ void fwd_group(int grow, GroupLds<D>& L, const u32x4* __restrict__ qc,
                                          const u32x4* __restrict__ kc, const u32x4* __restrict__ vc,
                                          const int32_t* __restrict__ lut, const int32_t* __restrict__ counts,
                                          int cap, const Geom& g, float sc_log2, bf16* __restrict__ oc,
                                          float* __restrict__ lse_c, int ngroups, const CubeDiv& cd,
                                          int dense_div) {
  constexpr int NDS = D / 16, NDT = D / 32, BLK = 64 * D / 8;
  constexpr int PER_WAVE = 2 * BLK / 64 / kGroup;   // 1 KB copies per wave per tile (K then V)
  auto& ring = L.ring;
  auto& ulist = L.ulist;
  auto& bits = L.bits;
  auto& wpre = L.wpre;
  auto& flag_bad = L.flag_bad;
  const long long bh = grow / ngroups;
  const int i0 = (grow - (int)(bh * ngroups)) * kGroup;
  if (!group_dense(counts, cap, g.nblk, bh, i0, dense_div)) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int i = i0 + wave;
  const bool active = i < g.nblk;
  const int nwords = (g.nblk + 31) / 32;

  // ---- union of the group's lists, in LDS -------------------------------
  for (int t = threadIdx.x; t < kGroup * (kMaxBlocks / 32); t += 64 * kGroup) (&bits[0][0])[t] = 0u;
  if (threadIdx.x == 0) flag_bad = 0;
  __syncthreads();
  int count = 0;
  const int32_t* lrow = lut + (bh * g.nblk + i) * (long long)cap;
  if (active) {
    count = counts[bh * g.nblk + i];
    count = count < 0 ? 0 : (count > cap ? cap : count);
  }
  bool bad = false;
  for (int e = lane; e < count; e += 64) {
    const int j = lrow[e];
    const int jn = e + 1 < count ? lrow[e + 1] : g.nblk;
    bad |= j < 0 || j >= g.nblk || jn <= j;
    if (j >= 0 && j < g.nblk) atomicOr(&bits[wave][j >> 5], 1u << (j & 31));
  }
  if (__any(bad) && lane == 0) flag_bad = 1;
  __syncthreads();
  if (flag_bad) {   // not strictly ascending ids: each wave runs its own row
    if (active) fwd_row<D, TOK>((int)(bh * g.nblk + i), qc, kc, vc, lut, counts, cap, g, sc_log2, oc, lse_c, cd, 0);
    return;
  }
  // word t of the union: its population goes to wpre[t + 1], then a scan
  for (int t = threadIdx.x; t < nwords; t += 64 * kGroup) {
    uint32_t u = 0;
#pragma unroll
    for (int w = 0; w < kGroup; ++w) u |= bits[w][t];
    wpre[t + 1] = __popc(u);
  }
  if (threadIdx.x == 0) wpre[0] = 0;
  __syncthreads();
  if (wave == 0) {   // inclusive scan of wpre[1 .. nwords], 64 words per pass
    int carry = 0;
    for (int t0 = 0; t0 < nwords; t0 += 64) {
      const int t = t0 + lane;
      int v = t < nwords ? wpre[t + 1] : 0;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(v, o, 64);
        v += lane >= o ? y : 0;
      }
      if (t < nwords) wpre[t + 1] = v + carry;
      carry += __shfl(v, 63, 64);
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < nwords; t += 64 * kGroup) {
    uint32_t u = 0;
#pragma unroll
    for (int w = 0; w < kGroup; ++w) u |= bits[w][t];
    int pos = wpre[t];
    while (u) {
      const int b = __ffs(u) - 1;
      u &= u - 1;
      int mask = 0;
#pragma unroll
      for (int w = 0; w < kGroup; ++w) mask |= ((bits[w][t] >> b) & 1u) << w;
      ulist[pos++] = (32 * t + b) | (mask << 16);
    }
  }
  __syncthreads();
  const int U = wpre[nwords];

  // ---- per-wave state and the union walk ---------------------------------
  using RS = RowState<D>;
  constexpr int G1 = RS::G1, G2 = RS::G2;
  const int hf = lane >> 5, r = lane & 31;
  const int sig = 16 * (r >> 4) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
  const int kpos = hf * 32 + sig;
  const long long head = bh * (g.n_pad / 64) * (long long)BLK;
  const u32x4* kh = kc + head;
  const u32x4* vh = vc + head;
  RS S;
  {
    const u32x4* qb = qc + head + (long long)(active ? i : 0) * BLK;
#pragma unroll
    for (int c = 0; c < 2 * NDS; ++c) S.qreg[c] = qb[c * 64 + lane];
  }
  S.init(g, cd, sc_log2, lane);

  // copies of entry e into slot e % kSlots: wave w takes the 1 KB chunks
  // [w PER_WAVE, (w + 1) PER_WAVE) of the K tile followed by the V tile
  const uint32_t ring0 = (uint32_t)(size_t)(__attribute__((address_space(3))) const char*)(const char*)&ring[0][0];
  const uint32_t lane16 = 16u * (uint32_t)lane;
  auto issue = [&](int e) {
    const int j = __builtin_amdgcn_readfirstlane(ulist[e] & 0xffff);
    const u32x4* kb = kh + (long long)j * BLK;
    const u32x4* vb = vh + (long long)j * BLK;
    const uint32_t dst = ring0 + (uint32_t)((e % kSlots) * 2 * BLK * 16);
#pragma unroll
    for (int c = 0; c < PER_WAVE; ++c) {
      const int ch = wave * PER_WAVE + c;   // chunk of the 2 BLK / 64 in the slot
      const u32x4* src = ch < BLK / 64 ? kb + ch * 64 : vb + (ch - BLK / 64) * 64;
      chunk_to_lds(dst + (uint32_t)(ch * 1024), src, lane16);
    }
  };
  // everything loaded so far (lists, counts, Q) has landed before the first
  // copy is queued, so the waits below count copies only
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
#pragma unroll
  for (int e = 0; e < kSlots - 1; ++e)
    if (e < U) issue(e);
  f32x16 stA[2], stB[2];
  uint32_t pA[2][8], pB[2][8];
  for (int u = 0; u < U; ++u) {
    // this entry's copies are done once only the later entries' remain
    const int later = min(U - 1 - u, kSlots - 2);
    if (later >= 2)
      __builtin_amdgcn_s_waitcnt(wait_vm(2 * PER_WAVE));
    else if (later == 1)
      __builtin_amdgcn_s_waitcnt(wait_vm(PER_WAVE));
    else
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
    // every wave's copies of this entry have landed, and every wave is done
    // with the slot the next copy refills
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (u + kSlots - 1 < U) issue(u + kSlots - 1);
    const int ent = ulist[u];
    if (!((ent >> (16 + wave)) & 1)) continue;
    const int j = ent & 0xffff;
    // the block step of fwd_row, with the operands read from LDS
    const u32x4* ks = &ring[u % kSlots][0];
    const u32x4* vs = ks + BLK;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) S.kreg[kt][ds] = ks[(kt * NDS + ds) * 64 + kpos];
    const uint64_t real = S.real_mask(j);
    S.gemm1_half(0, stA, real);
    {
      const float nmu = S.neg_m(0);
      float ls = 0.f;
      S.gemm1_first(stB, S.qchunk(1, 0), real);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k + 2 < G1) S.gemm1_step(stB, S.qchunk(1, (k + 2) >> 1), k + 2);
        S.exp_pair(stA, pA, nmu, ls, k);
        __builtin_amdgcn_sched_barrier(0);
      }
      RS::pin(pA);
#pragma unroll
      for (int ks4 = 0; ks4 < 4; ++ks4)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) S.vreg[dt][ks4] = vs[(dt * 4 + ks4) * 64 + lane];
      S.settle(0, stA, pA, ls);
    }
    {
      const float nmu = S.neg_m(1);
      float ls = 0.f;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k < G2) S.gemm2_step(0, pA, k);
        S.exp_pair(stB, pB, nmu, ls, k);
        __builtin_amdgcn_sched_barrier(0);
      }
      RS::pin(pB);
      S.settle(1, stB, pB, ls);
    }
#pragma unroll
    for (int k = 0; k < G2; ++k) S.gemm2_step(1, pB, k);
  }
  if (active) S.template epilogue<TOK>(bh, i, r, oc, lse_c);
}

// One workgroup per group (row of the group map).
template <int D, bool TOK>
__global__ __launch_bounds__(64 * kGroup) void fwd_group_kernel(
    const u32x4* __restrict__ qc, const u32x4* __restrict__ kc, const u32x4* __restrict__ vc,
    const int32_t* __restrict__ lut, const int32_t* __restrict__ counts, int cap, Geom g, float sc_log2,
    bf16* __restrict__ oc, float* __restrict__ lse_c, RowMap map, int ngroups, CubeDiv cd, int dense_div) {
  __shared__ GroupLds<D> L;
  const int grow = row_of_workgroup(blockIdx.x, map);
  if (grow < 0) return;
  fwd_group<D, TOK>(grow, L, qc, kc, vc, lut, counts, cap, g, sc_log2, oc, lse_c, ngroups, cd, dense_div);
}

// One workgroup per row: workgroups are dispatched round-robin over the 8
// XCDs, and the row map gives each XCD a contiguous run of rows so
// neighbouring query blocks (overlapping lists) share K/V tiles in its L2.
// With `order` (written by fwd_sched_kernel), workgroup w runs row
// order[(w % 8) * per_xcd + w / 8] instead.  With dense_div > 0 the rows of
// dense groups are left to fwd_group_kernel.
template <int D, bool TOK>
__global__ __launch_bounds__(64) void fwd_kernel(const u32x4* __restrict__ qc, const u32x4* __restrict__ kc,
                                                 const u32x4* __restrict__ vc, const int32_t* __restrict__ lut,
                                                 const int32_t* __restrict__ counts, int cap, Geom g,
                                                 float sc_log2, bf16* __restrict__ oc, float* __restrict__ lse_c,
                                                 RowMap map, CubeDiv cd, int qg_shift,
                                                 const int32_t* __restrict__ order, int dense_div) {
  const int row = order != nullptr
                      ? order[(long long)(blockIdx.x % kXcds) * map.per_xcd + blockIdx.x / kXcds]
                      : row_of_workgroup(blockIdx.x, map);
  if (row < 0) return;
  fwd_row<D, TOK>(row, qc, kc, vc, lut, counts, cap, g, sc_log2, oc, lse_c, cd, qg_shift, dense_div);
}

// ---------------------------------------------------------------------------
// Count-balanced row order.
//
// Rows have lists of different lengths.  When they differ little (Top-p and
// Top-k keep 1 to 1.3 times the mean of a quarter head on the 720p
// workloads), the hardware dispatcher balances them by itself: each SIMD takes
// the next workgroup as soon as its row ends, and the sweep order keeps
// neighbouring query blocks (overlapping lists) together in an XCD's L2.
// When they differ a lot (per-row budgets spread over two orders of
// magnitude), a long row dispatched late ends well after the others.  The
// schedule kernel therefore writes the order in which each XCD's workgroups
// take their rows: the row map's sweep, with each run of rows (a quarter of a
// head) whose longest list exceeds twice the run's mean reordered longest
// first, so that such a run ends with its shortest rows.  (A persistent grid
// of resident wavefronts pulling rows from per-XCD queues in the same orders
// was measured slower than hardware dispatch on every workload.)

constexpr int kSortMax = 1024;   // rows sorted together (a longer run is split)

struct SchedDims {
  int per_xcd;   // workgroups per XCD
  int chunk;     // rows per run (the row map's chunk, at most kSortMax)
};

inline SchedDims sched_dims(const RowMap& m) {
  SchedDims s;
  s.per_xcd = m.per_xcd;
  s.chunk = m.chunk < kSortMax ? m.chunk : kSortMax;
  return s;
}

// order[x * per_xcd + k] = the row of the k-th workgroup of XCD x (-1:
// none).  One workgroup of 256 threads per (run, XCD).
__global__ __launch_bounds__(256) void fwd_sched_kernel(const int32_t* __restrict__ counts, int cap, RowMap map,
                                                        SchedDims sd, int nblk, int32_t* __restrict__ order) {
  __shared__ int key[kSortMax];
  __shared__ int rowv[kSortMax];
  __shared__ int redm[4];
  __shared__ long long reds[4];
  const int x = blockIdx.y;
  const int k0 = blockIdx.x * sd.chunk;
  const int n = min(sd.chunk, sd.per_xcd - k0);
  int mx = 0;
  long long sum = 0;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int row = row_of_workgroup(x + kXcds * (k0 + e), map);
    int c = -1;
    if (row >= 0) {
      c = counts[row];
      c = c < 0 ? 0 : (c > cap ? cap : c);
      mx = max(mx, c);
      sum += c;
    }
    key[e] = c;
    rowv[e] = row;
  }
  // longest list and total of the run
  mx = max(mx, __shfl_xor(mx, 32));
  sum += __shfl_xor(sum, 32);
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) {
    mx = max(mx, __shfl_xor(mx, o));
    sum += __shfl_xor(sum, o);
  }
  if ((threadIdx.x & 63) == 0) {
    redm[threadIdx.x >> 6] = mx;
    reds[threadIdx.x >> 6] = sum;
  }
  __syncthreads();
  mx = max(max(redm[0], redm[1]), max(redm[2], redm[3]));
  const long long total = reds[0] + reds[1] + reds[2] + reds[3];
  const bool sort = (long long)mx * n > 2 * total;   // longest above twice the mean
  int32_t* out = order + (long long)x * sd.per_xcd + k0;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    int rank = e;
    if (sort) {   // count descending, then position in the sweep
      const int ke = key[e];
      rank = 0;
      for (int f = 0; f < n; ++f) {
        const int kf = key[f];
        rank += (kf > ke || (kf == ke && f < e)) ? 1 : 0;
      }
    }
    out[rank] = rowv[e];
  }
}

}  // namespace

size_t fwd_workspace_bytes(const Geom& g) {
  const RowMap map = make_rowmap(g.nblk, g.batch * g.heads);
  return ((size_t)kXcds * map.per_xcd * sizeof(int32_t) + 255) / 256 * 256;
}

// order: NULL (the row map's sweep) or a workspace for the count-balanced
// order (one list per cube only)
template <bool TOK>
static hipError_t launch_fwd_any(const void* qc, const void* kc, const void* vc, const int32_t* lut,
                                 const int32_t* counts, int cap, const Geom& g, float scale, void* out,
                                 float* lse_out, hipStream_t s, int qg_shift, void* order_ws, int max_count) {
  const RowMap map = make_rowmap(g.nblk, g.batch * g.heads);
  const CubeDiv cd = {make_fastdiv((uint32_t)g.nw), make_fastdiv((uint32_t)g.nh)};
  const float sc_log2 = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)((long long)map.per_xcd * kXcds));
  int32_t* order = qg_shift == 0 ? static_cast<int32_t*>(order_ws) : nullptr;
  if (order != nullptr) {
    const SchedDims sd = sched_dims(map);
    const dim3 sgrid((unsigned)((map.per_xcd + sd.chunk - 1) / sd.chunk), kXcds);
    fwd_sched_kernel<<<sgrid, 256, 0, s>>>(counts, cap, map, sd, g.nblk, order);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const u32x4* q = static_cast<const u32x4*>(qc);
  const u32x4* k = static_cast<const u32x4*>(kc);
  const u32x4* v = static_cast<const u32x4*>(vc);
  // dense groups go to the LDS-sharing kernel (one list per cube only), where a
  // head's K/V is too large for the L2 of the four XCDs that sweep it (16 MB):
  // there the one-wave kernel's dense sweeps run from beyond L2 (720p: 46 MB per
  // head, 0.27 of the bf16 peak against 0.35 for the group kernel), while with
  // smaller heads it keeps up (480p: 20 MB, 0.39 against 0.35)
  const size_t kv_head = (size_t)g.nblk * 64 * g.d * 2 * 2;
  // (and a known bound on the list lengths can rule dense groups out: a group
  // is dense only when its mean list reaches nblk / kDenseDiv)
  const bool maybe_dense = max_count < 0 || (long long)max_count * kDenseDiv >= g.nblk;
  const int dense_div =
      (qg_shift == 0 && g.nblk <= kMaxBlocks && kv_head >= kDenseHeadBytes && maybe_dense) ? kDenseDiv : 0;
  bf16* o = static_cast<bf16*>(out);
  if (g.d == 128)
    fwd_kernel<128, TOK><<<grid, 64, 0, s>>>(q, k, v, lut, counts, cap, g, sc_log2, o, lse_out, map, cd, qg_shift,
                                             order, dense_div);
  else
    fwd_kernel<64, TOK><<<grid, 64, 0, s>>>(q, k, v, lut, counts, cap, g, sc_log2, o, lse_out, map, cd, qg_shift,
                                            order, dense_div);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || dense_div == 0) return e;
  const int ngroups = (g.nblk + kGroup - 1) / kGroup;
  const RowMap gmap = make_rowmap(ngroups, g.batch * g.heads);
  const dim3 ggrid((unsigned)((long long)gmap.per_xcd * kXcds));
  if (g.d == 128)
    fwd_group_kernel<128, TOK><<<ggrid, 64 * kGroup, 0, s>>>(q, k, v, lut, counts, cap, g, sc_log2, o, lse_out,
                                                             gmap, ngroups, cd, dense_div);
  else
    fwd_group_kernel<64, TOK><<<ggrid, 64 * kGroup, 0, s>>>(q, k, v, lut, counts, cap, g, sc_log2, o, lse_out,
                                                            gmap, ngroups, cd, dense_div);
  return hipGetLastError();
}

hipError_t launch_fwd(const void* qc, const void* kc, const void* vc, const int32_t* lut,
                      const int32_t* counts, int cap, const Geom& g, float scale, void* oc,
                      float* lse_c, void* workspace, hipStream_t s, int qg_shift, int max_count) {
  return launch_fwd_any<false>(qc, kc, vc, lut, counts, cap, g, scale, oc, lse_c, s, qg_shift, workspace,
                               max_count);
}

hipError_t launch_fwd_tokens(const void* qc, const void* kc, const void* vc, const int32_t* lut,
                             const int32_t* counts, int cap, const Geom& g, float scale, void* o,
                             float* lse, hipStream_t s, void* workspace, int max_count) {
  return launch_fwd_any<true>(qc, kc, vc, lut, counts, cap, g, scale, o, lse, s, 0, workspace, max_count);
}

}  // namespace sa
