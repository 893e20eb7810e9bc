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

// TOK = false: O and LSE slot-major (oc [.., n_pad, D], lse_c [.., n_pad]);
// TOK = true: straight to token order (o [.., N, D], lse [.., N]), pad slots
// not written -- the inverse re-indexing fused into the epilogue.
// One query block (row of batch*heads*nblk) of the forward, by one wavefront.
template <int D, bool TOK>
__device__ __forceinline__ void fwd_row(int row, const u32x4* __restrict__ qc, const u32x4* __restrict__ kc,
                                        const u32x4* __restrict__ vc, const int32_t* __restrict__ lut,
                                        const int32_t* __restrict__ counts, int cap, const Geom& g,
                                        float sc_log2, bf16* __restrict__ oc, float* __restrict__ lse_c,
                                        const CubeDiv& cd, int qg_shift) {
  constexpr int NDS = D / 16;     // 16-dim steps of S^T
  constexpr int NDT = D / 32;     // 32-dim tiles of O^T
  constexpr int BLK = 64 * D / 8; // 16-byte units per block

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

  // Q^T operand chunks, in registers for the whole row
  u32x4 qreg[2 * NDS];
#pragma unroll
  for (int c = 0; c < 2 * NDS; ++c) qreg[c] = qb[c * 64 + lane];

  // the list of this query block: one per cube, or one per group of
  // 2^qg_shift consecutive cubes (asymmetric query blocks)
  const int nlists = (g.nblk + (1 << qg_shift) - 1) >> qg_shift;
  const long long lrow_i = bh * nlists + (i >> qg_shift);
  int count = counts[lrow_i];
  count = count < 0 ? 0 : (count > cap ? cap : count);
  const int32_t* lrow = lut + lrow_i * cap;

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
  // slot offsets of this lane's key slot, fixed for the whole row
  int lt, lh, lw;
  slot_offsets(g, lane, lt, lh, lw);
  // bit s set iff slot s of block j holds a real token; the cube coordinates
  // are uniform (scalar unit), only partial cubes need a per-lane test
  auto real_mask = [&](int j) -> uint64_t {
    const bool ok = valid_id(j);
    const uint32_t jj = ok ? (uint32_t)j : 0u;
    const uint32_t r = fdiv(jj, cd.w);
    const int bw = (int)jj - (int)r * g.nw;
    const int bt = (int)fdiv(r, cd.h);
    const int bh = (int)r - bt * g.nh;
    const int rt = min(g.ct, g.frames - bt * g.ct);
    const int rh = min(g.ch, g.height - bh * g.ch);
    const int rw = min(g.cw, g.width - bw * g.cw);
    const uint64_t b = ballot(lt < rt && lh < rh && lw < rw);
    return ok ? b : 0ull;
  };
  // both tiles are requested in the order the products consume them, so a
  // product waits only for the chunks it uses
  auto load_k = [&](int j) {
    const u32x4* kb = kh + (long long)(valid_id(j) ? j : 0) * BLK;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) kreg[kt][ds] = kb[(kt * NDS + ds) * 64 + kpos];
  };
  auto load_v = [&](int j) {
    const u32x4* vb = vh + (long long)(valid_id(j) ? j : 0) * BLK;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vreg[dt][ks] = vb[(dt * 4 + ks) * 64 + lane];
  };

  auto lane_mask = [&](uint64_t real) -> uint32_t {
    // this lane's 32 key bits: byte (kt, g) = keys 32 kt + 16 g + 8 hf .. +7
    return (uint32_t)((real >> (8 * hf)) & 0xffu) | ((uint32_t)((real >> (16 + 8 * hf)) & 0xffu) << 8) |
           ((uint32_t)((real >> (32 + 8 * hf)) & 0xffu) << 16) |
           ((uint32_t)((real >> (48 + 8 * hf)) & 0xffu) << 24);
  };  constexpr int G1 = 2 * NDS;       // MFMA steps of S^T for one half
  constexpr int G2 = 4 * NDT;       // MFMA steps of O^T for one half

  // ---- stages of one block, for one 32-query half qt ---------------------
  // S^T = K Q^T, one MFMA per step (16 steps: ds = step / 2, kt = step % 2);
  // q holds the Q^T chunk of this step's ds
  auto gemm1_step = [&](f32x16 (&st)[2], const u32x4& q, int step) {
    const int ds = step >> 1, kt = step & 1;
    st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[kt][ds]), as_bf16x8(q), st[kt], 0, 0, 0);
  };
  auto qchunk = [&](int qt, int ds) { return qreg[qt * NDS + ds]; };
  // Register e of tile kt holds key 32 kt + 16 (e / 8) + 8 hf + e % 8, i.e.
  // bit 16 kt + e of the lane's key mask.  Pad keys of a partial block get
  // S = -inf (so P = 0 and they never set the max) by starting their
  // accumulators at -inf instead of 0: the first MFMA of each tile reads the
  // start value, so a full block (wave-uniform branch) keeps the free zero
  // operand and a partial one pays 32 selects that wait on nothing.
  auto gemm1_first = [&](f32x16 (&st)[2], const u32x4& q, uint64_t real) {
    if (real == ~0ull) {
      const f32x16 z = {};
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[kt][0]), as_bf16x8(q), z, 0, 0, 0);
    } else {
      uint32_t lm = lane_mask(real);
      asm volatile("" : "+v"(lm));
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x16 init;
#pragma unroll
        for (int e = 0; e < 16; ++e) init[e] = ((lm >> (16 * kt + e)) & 1u) ? 0.f : -INFINITY;
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[kt][0]), as_bf16x8(q), init, 0, 0, 0);
      }
    }
  };
  // the whole S^T half in one region
  auto gemm1_half = [&](int qt, f32x16 (&st)[2], uint64_t real) {
    gemm1_first(st, qchunk(qt, 0), real);
#pragma unroll
    for (int k = 2; k < G1; ++k) gemm1_step(st, qchunk(qt, k >> 1), k);
  };
  // one register pair of P = exp2(scale S - m) (bf16-packed) and its sum
  auto exp_pair = [&](const f32x16 (&st)[2], uint32_t (&pw)[2][8], float nmu, float& ls, int step) {
    const int kt = step >> 3, e = 2 * (step & 7);
    const float p0 = __builtin_amdgcn_exp2f(fmaf(st[kt][e], sc_log2, nmu));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(st[kt][e + 1], sc_log2, nmu));
    ls += p0 + p1;
    pw[kt][e >> 1] = pack_bf16x2(p0, p1);
  };
  // row max of one half (raw scores; the scale is positive)
  auto half_max = [&](const f32x16 (&st)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, st[kt][e]);
    // the two half-waves hold the two halves of every query's keys
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sc_log2;
  };
  // O^T += V^T P^T, one MFMA per step (16 steps: ks = step / NDT, dt =
  // step % NDT at d = 128); k-step ks covers keys 16 ks .. +15 = registers
  // 8 (ks % 2) .. +7 of tile ks / 2
  auto gemm2_step = [&](int qt, const uint32_t (&pw)[2][8], int step) {
    const int ks = step / NDT, dt = step % NDT;
    const int kt = ks >> 1, o4 = 4 * (ks & 1);
    const u32x4 bw = {pw[kt][o4], pw[kt][o4 + 1], pw[kt][o4 + 2], pw[kt][o4 + 3]};
    acc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vreg[dt][ks]), as_bf16x8(bw), acc[dt][qt],
                                                          0, 0, 0);
  };

  // empty asm "uses": keep a stage's results computed in its own region (the
  // compiler would otherwise sink the softmax past the next branch and lose
  // the overlap with the matrix cores)
  auto pin = [](const uint32_t (&pw)[2][8]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 8; ++e) asm volatile("" ::"v"(pw[kt][e]));
  };
  // The exponentials of a half are computed with the current m right away and
  // checked afterwards through their sum; the rare half whose sum exceeds the
  // limit, or that finds m unset (always the first block), takes the exact
  // max, raises m, rescales the accumulator and is redone with the new m.
  auto settle = [&](int qt, const f32x16 (&st)[2], uint32_t (&pw)[2][8], float& ls) {
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
  };
  auto neg_m = [&](int qt) { return m[qt] == -INFINITY ? 0.f : -m[qt]; };
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
    real = real_mask(j_cur);
    gemm1_half(0, stA, real);
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
      const float nmu = neg_m(0);
      float ls = 0.f;
      gemm1_first(stB, qchunk(1, 0), real);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k + 2 < G1) gemm1_step(stB, qchunk(1, (k + 2) >> 1), k + 2);
        exp_pair(stA, pA, nmu, ls, k);
        __builtin_amdgcn_sched_barrier(0);
      }
      pin(pA);
      load_k(j_next);
      settle(0, stA, pA, ls);
    }
    {
      const float nmu = neg_m(1);
      float ls = 0.f;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k < G2) gemm2_step(0, pA, k);
        exp_pair(stB, pB, nmu, ls, k);
        if (k == 4) real_next = real_mask(j_next);   // scalar work between matrix ops
        __builtin_amdgcn_sched_barrier(0);
      }
      pin(pB);
      settle(1, stB, pB, ls);
    }
#pragma unroll
    for (int k = 0; k < G2; ++k) gemm2_step(1, pB, k);
    real = real_next;
    gemm1_half(0, stA, real);
    load_v(j_next);
    j_cur = j_next;
  }

  // epilogue: O = acc / l, LSE = (m + log2 l) ln 2; pad queries and empty rows -> 0, -inf
  const uint64_t qreal = real_mask(i);
  bf16* ob = oc + (bh * g.n_pad + (long long)i * 64) * D;
  float* lb = lse_c + bh * g.n_pad + (long long)i * 64;
  // token order: cube coordinates of this query block (one division each on the scalar unit)
  int ct0 = 0, ch0 = 0, cw0 = 0;
  if (TOK) {
    const uint32_t rr = fdiv((uint32_t)i, cd.w);
    cw0 = (i - (int)rr * g.nw) * g.cw;
    const int bt = (int)fdiv(rr, cd.h);
    ch0 = ((int)rr - bt * g.nh) * g.ch;
    ct0 = bt * g.ct;
  }
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float lt = l[qt] + __shfl_xor(l[qt], 32, 64);
    const int q = 32 * qt + r;
    const bool real_q = (qreal >> q) & 1ull;
    const bool live = real_q && lt > 0.f;
    const float inv = live ? 1.f / lt : 0.f;
    bf16* orow = ob + (long long)q * D;
    long long tok = 0;
    if (TOK) {
      int tt, hh, ww;
      slot_offsets(g, q, tt, hh, ww);
      tok = ((long long)(ct0 + tt) * g.height + (ch0 + hh)) * g.width + (cw0 + ww);
      orow = oc + (bh * g.n_real + tok) * D;
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
    const float lse_q = live ? (m[qt] + __log2f(lt)) * kLn2 : -INFINITY;
    if (hf == 0) {
      if (TOK)
        lse_c[bh * g.n_real + tok] = lse_q;
      else
        lb[q] = lse_q;
    }
  }
}

// One workgroup per row: workgroups are dispatched round-robin over the 8
// XCDs, and the row map gives each XCD a contiguous run of rows so
// neighbouring query blocks (overlapping lists) share K/V tiles in its L2.
// With `order` (written by fwd_sched_kernel), workgroup w runs row
// order[(w % 8) * per_xcd + w / 8] instead.
template <int D, bool TOK>
__global__ __launch_bounds__(64) void fwd_kernel(const u32x4* __restrict__ qc, const u32x4* __restrict__ kc,
                                                 const u32x4* __restrict__ vc, const int32_t* __restrict__ lut,
                                                 const int32_t* __restrict__ counts, int cap, Geom g,
                                                 float sc_log2, bf16* __restrict__ oc, float* __restrict__ lse_c,
                                                 RowMap map, CubeDiv cd, int qg_shift,
                                                 const int32_t* __restrict__ order) {
  const int row = order != nullptr
                      ? order[(long long)(blockIdx.x % kXcds) * map.per_xcd + blockIdx.x / kXcds]
                      : row_of_workgroup(blockIdx.x, map);
  if (row < 0) return;
  fwd_row<D, TOK>(row, qc, kc, vc, lut, counts, cap, g, sc_log2, oc, lse_c, cd, qg_shift);
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
                                 float* lse_out, hipStream_t s, int qg_shift, void* order_ws) {
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
  if (g.d == 128)
    fwd_kernel<128, TOK><<<grid, 64, 0, s>>>(q, k, v, lut, counts, cap, g, sc_log2, static_cast<bf16*>(out),
                                             lse_out, map, cd, qg_shift, order);
  else
    fwd_kernel<64, TOK><<<grid, 64, 0, s>>>(q, k, v, lut, counts, cap, g, sc_log2, static_cast<bf16*>(out),
                                            lse_out, map, cd, qg_shift, order);
  return hipGetLastError();
}

hipError_t launch_fwd(const void* qc, const void* kc, const void* vc, const int32_t* lut,
                      const int32_t* counts, int cap, const Geom& g, float scale, void* oc,
                      float* lse_c, void* workspace, hipStream_t s, int qg_shift) {
  return launch_fwd_any<false>(qc, kc, vc, lut, counts, cap, g, scale, oc, lse_c, s, qg_shift, workspace);
}

hipError_t launch_fwd_tokens(const void* qc, const void* kc, const void* vc, const int32_t* lut,
                             const int32_t* counts, int cap, const Geom& g, float scale, void* o,
                             float* lse, hipStream_t s, void* workspace) {
  return launch_fwd_any<true>(qc, kc, vc, lut, counts, cap, g, scale, o, lse, s, 0, workspace);
}

}  // namespace sa
