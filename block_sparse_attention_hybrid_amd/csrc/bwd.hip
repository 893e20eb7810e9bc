// Backward pass of the block-sparse attention (gfx950).
//
// SpargeAttention2 summary page, "Why this implementation is trainable": the
// kernel must carry gradients through the kept blocks (the mask itself has
// none).  For query block i with kept key blocks j, with P recomputed from the
// saved log-sum-exp,
//   D = rowsum(dO * O),  dP = dO V^T,  dS = P * (dP - D),
//   dV_j += P^T dO,  dK_j += scale dS^T Q,  dQ_i += scale dS K.
// Two kernels avoid atomics and keep the result deterministic:
//   * dq: one wavefront per query block walks the block's kept list (as the
//     forward does) and accumulates dQ^T = K^T dS^T in registers;
//   * dkv: one workgroup per key block walks the transposed list (the query
//     blocks that keep it, from sparse_attn_transpose_lut); each of its four
//     waves owns 32 of the block's keys and one query half and accumulates
//     dV^T = dO^T P and dK^T = Q^T dS in registers, reading the query
//     block's Q and dO from LDS, where the workgroup stages them once (in the
//     QK layout only: the products over queries read them transposed).
// Operand orders follow the forward kernel: every MFMA operand is one 16-byte
// chunk per lane of a QK- or V-layout block (sa_layout.h), and the rows fed
// to the first product are permuted (sigma) so that a lane's accumulator
// registers hold 8 consecutive tokens for each 16-token step of the second
// product, which then takes them straight from registers as bf16 pairs.
#include "sa_launch.h"
#include "sa_layout.h"
#include "sa_rowmap.h"

#include <math.h>

namespace sa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
#ifndef SA_DQ_XCD_GROUP
#define SA_DQ_XCD_GROUP 4
#endif
constexpr int kDqXcdGroup = SA_DQ_XCD_GROUP;   // XCDs sweeping one head together in the dq kernel

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Row r of a 32-row MFMA tile is fed token sigma(r) (see the forward kernel).
__device__ __forceinline__ int sigma32(int r) {
  return 16 * (r >> 4) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
}

// D = rowsum(dO * O) of every slot: one wavefront per block, lane = slot.
__global__ __launch_bounds__(64) void bwd_delta_kernel(const u32x4* __restrict__ oc,
                                                       const u32x4* __restrict__ do_qk,
                                                       float* __restrict__ delta, Geom g) {
  const int i = blockIdx.x;
  const long long bh = blockIdx.y;
  const int s = threadIdx.x, d = g.d, cpr = d / 8;
  const long long base = (bh * g.n_pad + (long long)i * kBlock) * cpr;
  float acc = 0.f;
  for (int c8 = 0; c8 < cpr; ++c8) {
    const u32x4 o = oc[base + (long long)s * cpr + c8];
    const u32x4 w = do_qk[base + qk_offset(s, 8 * c8, d) / 8];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += lo_bf16(o[e]) * lo_bf16(w[e]) + hi_bf16(o[e]) * hi_bf16(w[e]);
  }
  delta[bh * g.n_pad + (long long)i * kBlock + s] = acc;
}

__global__ void zero_words_kernel(uint32_t* __restrict__ p, long long n) {
  for (long long x = blockIdx.x * (long long)blockDim.x + threadIdx.x; x < n; x += (long long)gridDim.x * blockDim.x)
    p[x] = 0u;
}

// Bit i of row j of a head's bitmap: query block i keeps key block j.
__global__ __launch_bounds__(64) void lut_mark_kernel(const int32_t* __restrict__ lut,
                                                      const int32_t* __restrict__ counts, int cap,
                                                      uint32_t* __restrict__ bits, Geom g, int words) {
  const long long row = blockIdx.x;
  const long long bh = row / g.nblk;
  const int i = (int)(row - bh * g.nblk);
  int cnt = counts[row];
  cnt = cnt < 0 ? 0 : (cnt > cap ? cap : cnt);
  const int32_t* l = lut + row * cap;
  for (int e = threadIdx.x; e < cnt; e += 64) {
    const int j = l[e];
    if (j >= 0 && j < g.nblk) atomicOr(&bits[(bh * g.nblk + j) * words + (i >> 5)], 1u << (i & 31));
  }
}

// Ascending list of the query blocks that keep key block j (one wave per j).
__global__ __launch_bounds__(64) void lut_gather_kernel(const uint32_t* __restrict__ bits,
                                                        int32_t* __restrict__ lut_t,
                                                        int32_t* __restrict__ counts_t, int cap_t, int words) {
  const long long col = blockIdx.x;
  const int lane = threadIdx.x;
  const uint32_t* wrow = bits + col * words;
  int32_t* out = lut_t + col * cap_t;
  int written = 0;
  for (int w0 = 0; w0 < words; w0 += 64) {
    const int w = w0 + lane;
    uint32_t word = w < words ? wrow[w] : 0u;
    const int c = __popc(word);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    int pos = written + incl - c;
    while (word) {
      const int b = __ffs(word) - 1;
      word &= word - 1u;
      if (pos < cap_t) out[pos] = w * 32 + b;
      ++pos;
    }
    written += __shfl(incl, 63, 64);
  }
  if (lane == 0) counts_t[col] = written;
}

// Log2-domain LSE of a query slot: +inf for slots without attention (pad
// slots, empty rows), so that their recomputed probabilities are 0.
__device__ __forceinline__ float lse2_of(float lse) { return lse > -INFINITY ? lse * kLog2e : INFINITY; }

template <int D>
__global__ __launch_bounds__(64) void bwd_dq_kernel(const u32x4* __restrict__ q, const u32x4* __restrict__ k,
                                                    const u32x4* __restrict__ v_qk, const u32x4* __restrict__ k_v,
                                                    const u32x4* __restrict__ do_qk, const float* __restrict__ lse,
                                                    const float* __restrict__ delta, const int32_t* __restrict__ lut,
                                                    const int32_t* __restrict__ counts, int cap, Geom g,
                                                    float sc_log2, float scale, bf16* __restrict__ dq,
                                                    RowMap map) {
  constexpr int NDS = D / 16, NDT = D / 32, BLK = 64 * D / 8;
  // XCD-aware order: each XCD sweeps neighbouring query blocks of one head,
  // whose kept lists overlap, so more of their K/V tiles hit its L2
  const int wrow = row_of_workgroup<kDqXcdGroup>(blockIdx.x, map);
  if (wrow < 0) return;
  const long long bh = wrow / g.nblk;
  const int i = wrow - (int)(bh * g.nblk);
  const long long row = wrow;
  const int lane = threadIdx.x, hf = lane >> 5, r = lane & 31;
  const int kpos = hf * 32 + sigma32(r);
  const long long head = bh * (long long)g.nblk * BLK;

  __shared__ u32x4 qlds[2 * NDS * 64];
  __shared__ u32x4 dolds[2 * NDS * 64];
  const u32x4* qb = q + head + (long long)i * BLK;
  const u32x4* dob = do_qk + head + (long long)i * BLK;
#pragma unroll
  for (int c = 0; c < 2 * NDS; ++c) {
    qlds[c * 64 + lane] = qb[c * 64 + lane];
    dolds[c * 64 + lane] = dob[c * 64 + lane];
  }
  __syncthreads();
  float l2[2], dl[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const long long slot = bh * g.n_pad + (long long)i * kBlock + 32 * qt + r;
    l2[qt] = lse2_of(lse[slot]);
    dl[qt] = delta[slot];
  }

  f32x16 acc[NDT][2];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][qt][e] = 0.f;

  int count = counts[row];
  count = count < 0 ? 0 : (count > cap ? cap : count);
  const int32_t* lrow = lut + row * cap;

  // slot offsets of this lane's key slot, for the per-block padding ballot
  int lt, lh, lw;
  slot_offsets(g, lane, lt, lh, lw);

  // K and V (QK layout) of the current block, K in the V layout
  u32x4 kreg[2][NDS], vreg[2][NDS], kvreg[NDT][4];
  auto block_id = [&](int it) {
    const int j0 = lrow[it];
    return (j0 >= 0 && j0 < g.nblk) ? j0 : -1;
  };
  auto base_of = [&](int j) { return head + (long long)(j < 0 ? 0 : j) * BLK; };
  auto load_k = [&](int j) {
    const long long o = base_of(j);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) kreg[kt][ds] = k[o + (kt * NDS + ds) * 64 + kpos];
  };
  auto load_v = [&](int j) {
    const long long o = base_of(j);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) vreg[kt][ds] = v_qk[o + (kt * NDS + ds) * 64 + kpos];
  };
  auto load_kvv = [&](int j) {
    const long long o = base_of(j);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kvreg[dt][ks] = k_v[o + (dt * 4 + ks) * 64 + lane];
  };
  // S^T and dP^T of one query half: one product over d with K or V as the
  // A operand.  The first MFMA takes the start value: the free zero operand,
  // or for S^T of a block with pad keys 0 (real key) / -inf (pad key), so
  // that P = 0 on pad keys with no select per element.
  const f32x16 zero = {};
  // the B operands of one product (this half's Q or dO chunks) are read from
  // LDS together, ahead of the MFMAs, so the read latency is paid once
  auto read_ops = [&](const u32x4* ops, int qt, u32x4 (&b)[NDS]) {
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) b[ds] = ops[(qt * NDS + ds) * 64 + lane];
  };
  auto product_rest = [&](const u32x4 (&a)[2][NDS], const u32x4 (&b)[NDS], f32x16 (&acc2)[2]) {
#pragma unroll
    for (int ds = 1; ds < NDS; ++ds)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        acc2[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[kt][ds]), as_bf16x8(b[ds]), acc2[kt], 0, 0, 0);
  };
  auto scores_s = [&](int qt, f32x16 (&st)[2], uint64_t real, uint32_t lm) {
    u32x4 b[NDS];
    read_ops(qlds, qt, b);
    if (real == ~0ull) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[kt][0]), as_bf16x8(b[0]), zero, 0, 0, 0);
    } else {
      asm volatile("" : "+v"(lm));
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x16 init;
#pragma unroll
        for (int e = 0; e < 16; ++e) init[e] = ((lm >> (16 * kt + e)) & 1u) ? 0.f : -INFINITY;
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[kt][0]), as_bf16x8(b[0]), init, 0, 0, 0);
      }
    }
    product_rest(kreg, b, st);
  };
  auto scores_dp = [&](int qt, f32x16 (&dpt)[2]) {
    u32x4 b[NDS];
    read_ops(dolds, qt, b);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
      dpt[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vreg[kt][0]), as_bf16x8(b[0]), zero, 0, 0, 0);
    product_rest(vreg, b, dpt);
  };
  // dS^T = P^T * (dP^T - D) of one query half, as bf16 pairs
  auto grad_scores = [&](const f32x16 (&st)[2], const f32x16 (&dpt)[2], int qt, uint32_t (&dsw)[2][8]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        float v2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float p = __builtin_amdgcn_exp2f(fmaf(st[kt][e + u], sc_log2, -l2[qt]));
          v2[u] = p * (dpt[kt][e + u] - dl[qt]);
        }
        dsw[kt][e >> 1] = pack_bf16x2(v2[0], v2[1]);
      }
  };

  // Per kept block t, each operand's registers are refilled for block t+1
  // as soon as their last product of block t is issued: K after the two
  // score products, V after the two dP products, K_v after the dQ products.
  // Every load thereby has most of a block of work as lead time.  Past the
  // last block the "next" block is the current one again (a redundant
  // reload rather than a branch, which would make the compiler wait for
  // every load in flight where the paths meet).
  int j = count > 0 ? block_id(0) : -1;
  if (count > 0) {
    load_k(j);
    load_v(j);
    load_kvv(j);
  }
  for (int it = 0; it < count; ++it) {
    const bool more = it + 1 < count;
    const int jn = more ? block_id(it + 1) : j;
    const uint64_t real = j >= 0 ? block_real_mask_wave(g, j, lt, lh, lw) : 0ull;
    // this lane's 32 key bits: register e of tile kt <-> key 32 kt + 16 (e / 8) + 8 hf + e % 8
    const uint32_t lm = (uint32_t)((real >> (8 * hf)) & 0xffu) | ((uint32_t)((real >> (16 + 8 * hf)) & 0xffu) << 8) |
                        ((uint32_t)((real >> (32 + 8 * hf)) & 0xffu) << 16) |
                        ((uint32_t)((real >> (48 + 8 * hf)) & 0xffu) << 24);
    // Q and dO are read from LDS at each use rather than held in registers
    // across the loop, which leaves the registers to the operands in flight
    asm volatile("" ::: "memory");
    f32x16 st0[2], st1[2], dpt[2];
    uint32_t dsw[2][2][8];
    // (scheduling barriers keep each refill where it is written: the
    // compiler would otherwise sink it to the next use to save registers)
    scores_s(0, st0, real, lm);
    scores_s(1, st1, real, lm);
    __builtin_amdgcn_sched_barrier(0);
    load_k(jn);
    __builtin_amdgcn_sched_barrier(0);
    scores_dp(0, dpt);
    grad_scores(st0, dpt, 0, dsw[0]);
    scores_dp(1, dpt);
    __builtin_amdgcn_sched_barrier(0);
    load_v(jn);
    __builtin_amdgcn_sched_barrier(0);
    grad_scores(st1, dpt, 1, dsw[1]);
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int step = 0; step < 4 * NDT; ++step) {
        const int ks = step / NDT, dt = step % NDT;
        const int kt = ks >> 1, o4 = 4 * (ks & 1);
        const u32x4 bw = {dsw[qt][kt][o4], dsw[qt][kt][o4 + 1], dsw[qt][kt][o4 + 2], dsw[qt][kt][o4 + 3]};
        acc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kvreg[dt][ks]), as_bf16x8(bw), acc[dt][qt],
                                                              0, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);
    load_kvv(jn);
    __builtin_amdgcn_sched_barrier(0);
    j = jn;
  }
  bf16* ob = dq + (bh * g.n_pad + (long long)i * 64) * D;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    bf16* orow = ob + (long long)(32 * qt + r) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const u32x2 v = {pack_bf16x2(acc[dt][qt][4 * a] * scale, acc[dt][qt][4 * a + 1] * scale),
                         pack_bf16x2(acc[dt][qt][4 * a + 2] * scale, acc[dt][qt][4 * a + 3] * scale)};
        *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * a + 4 * hf) = v;
      }
  }
}

// Direct global-to-LDS copy, 16 bytes per lane: lane l's bytes land at
// dst + 16 l (dst wave-uniform).  The builtin exists only for the device; the
// host pass of this file sees an empty body.
__device__ __forceinline__ void copy_to_lds(const u32x4* src, u32x4* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
#else
  (void)src;
  (void)dst;
#endif
}

// s_waitcnt immediates: vmcnt(n) alone (expcnt and lgkmcnt at their maxima),
// and lgkmcnt(0) alone (vmcnt and expcnt at their maxima)
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kLgkm0 = 0xC07F;

// LDS transpose read (ds_read_b64_tr_b16), 8 bytes per lane.  Within each
// group of 16 lanes, result lane i receives as its element e the (i % 4)-th
// 16-bit value of the 8 bytes addressed by lane 4 e + i / 4 of the group (a
// probe on gfx950 checked this mapping).  byte_off is wave-uniform plus this
// lane's part; the host pass sees an empty body.
__device__ __forceinline__ u32x2 read_tr16(const u32x4* lds_base, int byte_off) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  typedef __attribute__((address_space(3))) char lds_char;
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((lds_char*)lds_base + byte_off));
  return __builtin_bit_cast(u32x2, r);
#else
  (void)lds_base;
  (void)byte_off;
  return u32x2{0u, 0u};
#endif
}

// One workgroup of 4 waves per key block j.  Wave w owns keys 32 (w % 2) ..
// +31 and query half w / 2 of every query block in j's transposed list, and
// accumulates dV^T = dO^T P and dK^T = Q^T dS for those keys over that half;
// the two halves are added in LDS at the end (fixed order).  The query
// block's Q and dO (QK layout, 32 KB at d = 128) and its LSE and D rows are
// copied into LDS with direct global-to-LDS loads, double buffered: the copy
// of the next block is in flight while the current one is used, with
// explicit vmcnt waits and barriers (no fence that would drain the copy in
// flight).  The second and third products contract over queries, so their A
// operands (dO^T and Q^T: 8 consecutive queries of one dim per lane) are
// formed from the same staged QK-layout data with LDS transpose reads, two
// per operand; no second copy of Q and dO is needed.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkv_kernel(const u32x4* __restrict__ q, const u32x4* __restrict__ k,
                                                      const u32x4* __restrict__ v_qk,
                                                      const u32x4* __restrict__ do_qk, const float* __restrict__ lse,
                                                      const float* __restrict__ delta,
                                                      const int32_t* __restrict__ lut_t,
                                                      const int32_t* __restrict__ counts_t, int cap_t, Geom g,
                                                      float sc_log2, float scale, bf16* __restrict__ dk,
                                                      bf16* __restrict__ dv) {
  constexpr int NDS = D / 16, NDT = D / 32, BLK = 64 * D / 8;
  constexpr int NARR = 2 * NDS;          // 1 KB chunks per array (= 4 * NDT)
  constexpr int NCH = 2 * NARR;          // chunks per query block: Q, dO (QK layout)
  constexpr int PER_WAVE = NCH / 4;      // chunk copies issued by each wave
  // (plain order: the transposed lists differ widely in length, and a static
  // split of contiguous key blocks over the XCDs leaves them unbalanced)
  const int j = blockIdx.x;
  const long long bh = blockIdx.y;
  const long long col = bh * g.nblk + j;
  // the wave index is uniform: keep it (and the copy addresses) on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, hf = lane >> 5, r = lane & 31;
  const int kh = wave & 1, qq = wave >> 1;
  const long long head = bh * (long long)g.nblk * BLK;

  // per buffer: the NCH operand chunks, then one chunk whose first 256 bytes
  // hold the LSE row and the next 256 bytes the D row.  Inside a staged
  // chunk the token slots are rotated: QK-layout slot (h, r) of a chunk of
  // dim step ds sits at LDS slot h*32 + (r + 4h + 8 (ds % 2)) % 32.  A
  // transpose read takes both halves of 8 tokens from the chunks of two
  // neighbouring dim steps; with the rotation each half-wave of it meets
  // every bank once (unrotated, the halves 512 bytes apart and the chunks
  // 1 KB apart fell on the same banks).
  __shared__ u32x4 stage[2][(NCH + 1) * 64];
  auto lds_slot = [](int ds_odd, int h, int rr) { return h * 32 + ((rr + 4 * h + 8 * ds_odd) & 31); };

  // this wave's 32 keys (B operands, chunk t32 = kh) and whether this lane's key is real
  u32x4 kreg[NDS], vreg[NDS];
  const u32x4* kb = k + head + (long long)j * BLK;
  const u32x4* vb = v_qk + head + (long long)j * BLK;
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    kreg[ds] = kb[(kh * NDS + ds) * 64 + lane];
    vreg[ds] = vb[(kh * NDS + ds) * 64 + lane];
  }
  // all ones for a real key, zero for a pad slot; opaque so that the
  // compiler blends with it instead of branching around the exponentials
  uint32_t key_bits = slot_token(g, j, 32 * kh + r) >= 0 ? 0xffffffffu : 0u;
  asm volatile("" : "+v"(key_bits));

  // Transpose-read addresses.  The A operand of k-step ks (16 queries) and
  // dim tile dt needs, in lane (r, hf), queries 16 ks + 8 hf .. +7 of dim
  // 32 dt + r.  Read h (h = 0, 1) delivers queries 16 ks + 8 hf + 4 h .. +3:
  // lane s = 16 gq + 4 e + m of group gq supplies the 8 bytes holding dims
  // 32 dt + 16 (gq % 2) + 4 m .. +3 of query 16 ks + 8 (gq / 2) + 4 h + e,
  // i.e. half m / 2 of token slot 16 (ks % 2) + 4 h + 8 (gq / 2) + e of
  // chunk ((ks / 2) NDS + 2 dt + gq % 2).  This wave's k-steps have
  // ks / 2 = qq, so the lane part depends on (ks % 2, h) only: four offsets.
  int tr_lane[2][2];
  {
    const int gq = lane >> 4, e = (lane >> 2) & 3, m = lane & 3;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        tr_lane[kk][h] = (gq & 1) * 1024 + lds_slot(gq & 1, m >> 1, 16 * kk + 4 * h + 8 * (gq >> 1) + e) * 16 +
                         8 * (m & 1);
  }
  auto tr_operand = [&](const u32x4* arr, int dt, int ks) {
    const int base = ((ks >> 1) * NDS + 2 * dt) * 1024;
    const u32x2 lo = read_tr16(arr, base + tr_lane[ks & 1][0]);
    const u32x2 hi = read_tr16(arr, base + tr_lane[ks & 1][1]);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };

  f32x16 adk[NDT], adv[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) adk[t][e] = adv[t][e] = 0.f;

  int count = counts_t[col];
  count = count < 0 ? 0 : (count > cap_t ? cap_t : count);
  const int32_t* list = lut_t + col * cap_t;
  auto valid = [&](int i) { return i >= 0 && i < g.nblk; };
  // copy query block list[it] into buffer b: waves 0 and 1 copy the two
  // halves of Q, waves 2 and 3 those of dO; wave 0 also copies the LSE and D
  // rows (one 16-byte-lane copy whose lanes 0-15 take the 64 LSE values and
  // lanes 16-31 the 64 D values; lanes 32-63 repeat them into a part of the
  // slot that is not read)
  static_assert(2 * PER_WAVE == NARR, "half an array per wave");
  static_assert(PER_WAVE % 2 == 0 && NDS % 2 == 0, "a copied chunk's dim-step parity is cc % 2");
  const u32x4* my_src = (wave < 2 ? q : do_qk) + (wave & 1) * PER_WAVE * 64;
  const u32x4* row_src = reinterpret_cast<const u32x4*>((lane & 16) ? delta : lse);
  // LDS slot `lane` of a chunk of dim-step parity o receives QK-layout slot
  // (h, (lane - 4h - 8o) % 32), h = lane / 32 (the inverse of lds_slot)
  const int src_slot[2] = {hf * 32 + ((r - 4 * hf) & 31), hf * 32 + ((r - 4 * hf - 8) & 31)};
  auto issue = [&](int b, int it) {
    const int i0 = list[it];
    const int i = valid(i0) ? i0 : 0;
    const long long ob = head + (long long)i * BLK;
#pragma unroll
    for (int cc = 0; cc < PER_WAVE; ++cc)
      copy_to_lds(my_src + ob + cc * 64 + src_slot[cc & 1], &stage[b][(wave * PER_WAVE + cc) * 64]);
    if (wave == 0)
      copy_to_lds(row_src + (bh * g.n_pad + (long long)i * kBlock) / 4 + (lane & 15), &stage[b][NCH * 64]);
  };

  // the key operands are in registers before any copy is queued behind them,
  // so no wait inside the loop has to cover them
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  if (count > 0) issue(0, 0);
  for (int it = 0; it < count; ++it) {
    const int b = it & 1;
    if (it + 1 < count) {
      issue(b ^ 1, it + 1);
      // this block's copies are done once only the next block's remain in flight
      if (wave == 0)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_WAVE + 1));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_WAVE));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __builtin_amdgcn_s_barrier();   // every wave's copies of buffer b have landed
    if (valid(list[it])) {
      const u32x4* qs = &stage[b][0];
      const u32x4* dos = &stage[b][NARR * 64];
      const float* lrow = reinterpret_cast<const float*>(&stage[b][NCH * 64]);
      f32x16 s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = dp[e] = 0.f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const int qpos = lds_slot(ds & 1, hf, sigma32(r));
        const u32x4 qa = qs[(qq * NDS + ds) * 64 + qpos];
        const u32x4 da = dos[(qq * NDS + ds) * 64 + qpos];
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa), as_bf16x8(kreg[ds]), s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(da), as_bf16x8(vreg[ds]), dp, 0, 0, 0);
      }
      // register e <-> query 32 qq + 16 (e / 8) + 8 hf + e % 8; the lane's column is its key
      uint32_t pw[8], dsw[8];
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        float pv[2], sv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int qi = 32 * qq + 16 * ((e + u) >> 3) + 8 * hf + ((e + u) & 7);
          // pad keys: exponent -inf (bit blend), so p = 0 with no branch around the exponential
          const uint32_t xb = __float_as_uint(fmaf(s[e + u], sc_log2, -lse2_of(lrow[qi])));
          const float p = __builtin_amdgcn_exp2f(__uint_as_float((xb & key_bits) | (0xff800000u & ~key_bits)));
          pv[u] = p;
          sv[u] = p * (dp[e + u] - lrow[kBlock + qi]);
        }
        pw[e >> 1] = pack_bf16x2(pv[0], pv[1]);
        dsw[e >> 1] = pack_bf16x2(sv[0], sv[1]);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ks = 2 * qq + kk;
        const u32x4 bp = {pw[4 * kk], pw[4 * kk + 1], pw[4 * kk + 2], pw[4 * kk + 3]};
        const u32x4 bs = {dsw[4 * kk], dsw[4 * kk + 1], dsw[4 * kk + 2], dsw[4 * kk + 3]};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          adv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(tr_operand(dos, dt, ks)), as_bf16x8(bp),
                                                            adv[dt], 0, 0, 0);
          adk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(tr_operand(qs, dt, ks)), as_bf16x8(bs),
                                                            adk[dt], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(kLgkm0);   // this wave's LDS reads are complete
    __builtin_amdgcn_s_barrier();         // ... and every wave's, before b is refilled
  }

  // query half 1 hands its partial sums to query half 0 through LDS
  float* red = reinterpret_cast<float*>(&stage[0][0]);   // 2 key halves x 2 NDT x 16 x 64 floats
  float* mine = red + (size_t)kh * (2 * NDT * 16 * 64);
  if (qq == 1) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        mine[((2 * dt) * 16 + e) * 64 + lane] = adk[dt][e];
        mine[((2 * dt + 1) * 16 + e) * 64 + lane] = adv[dt][e];
      }
  }
  __syncthreads();
  if (qq == 1) return;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      adk[dt][e] += mine[((2 * dt) * 16 + e) * 64 + lane];
      adv[dt][e] += mine[((2 * dt + 1) * 16 + e) * 64 + lane];
    }
  const long long orow = (bh * g.n_pad + (long long)j * 64 + 32 * kh + r) * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const u32x2 kv2 = {pack_bf16x2(adk[dt][4 * a] * scale, adk[dt][4 * a + 1] * scale),
                         pack_bf16x2(adk[dt][4 * a + 2] * scale, adk[dt][4 * a + 3] * scale)};
      const u32x2 vv2 = {pack_bf16x2(adv[dt][4 * a], adv[dt][4 * a + 1]),
                         pack_bf16x2(adv[dt][4 * a + 2], adv[dt][4 * a + 3])};
      *reinterpret_cast<u32x2*>(dk + orow + 32 * dt + 8 * a + 4 * hf) = kv2;
      *reinterpret_cast<u32x2*>(dv + orow + 32 * dt + 8 * a + 4 * hf) = vv2;
    }
}

}  // namespace

hipError_t launch_bwd_delta(const void* oc, const void* do_qk, float* delta, const Geom& g, hipStream_t s) {
  dim3 grid(g.nblk, g.batch * g.heads);
  bwd_delta_kernel<<<grid, 64, 0, s>>>(static_cast<const u32x4*>(oc), static_cast<const u32x4*>(do_qk), delta, g);
  return hipGetLastError();
}

size_t transpose_workspace_bytes(const Geom& g) {
  const size_t words = (size_t)(g.nblk + 31) / 32;
  return (size_t)g.batch * g.heads * g.nblk * words * sizeof(uint32_t);
}

hipError_t launch_transpose_lut(const int32_t* lut, const int32_t* counts, int cap, int32_t* lut_t,
                                int32_t* counts_t, int cap_t, const Geom& g, void* workspace, hipStream_t s) {
  const int words = (g.nblk + 31) / 32;
  const long long rows = (long long)g.batch * g.heads * g.nblk;
  uint32_t* bits = static_cast<uint32_t*>(workspace);
  const long long n = rows * words;
  const long long blocks = (n + 255) / 256;
  zero_words_kernel<<<(unsigned)(blocks < 65536 ? blocks : 65536), 256, 0, s>>>(bits, n);
  lut_mark_kernel<<<(unsigned)rows, 64, 0, s>>>(lut, counts, cap, bits, g, words);
  lut_gather_kernel<<<(unsigned)rows, 64, 0, s>>>(bits, lut_t, counts_t, cap_t, words);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, const Geom& g, float scale, void* dq, void* dk, void* dv, hipStream_t s) {
  const float sc_log2 = scale * kLog2e;
  const RowMap map = make_rowmap<kDqXcdGroup>(g.nblk, g.batch * g.heads);
  const dim3 grid((unsigned)((long long)map.per_xcd * kXcds));   // dq, XCD-aware
  const dim3 grid_kv(g.nblk, g.batch * g.heads);
  auto U = [](const void* p) { return static_cast<const u32x4*>(p); };
  if (g.d == 128) {
    bwd_dq_kernel<128><<<grid, 64, 0, s>>>(U(a.q), U(a.k), U(a.v_qk), U(a.k_v), U(a.do_qk), a.lse, a.delta, a.lut,
                                           a.counts, a.cap, g, sc_log2, scale, static_cast<bf16*>(dq), map);
    bwd_dkv_kernel<128><<<grid_kv, 256, 0, s>>>(U(a.q), U(a.k), U(a.v_qk), U(a.do_qk), a.lse,
                                             a.delta, a.lut_t, a.counts_t, a.cap_t, g, sc_log2, scale,
                                             static_cast<bf16*>(dk), static_cast<bf16*>(dv));
  } else {
    bwd_dq_kernel<64><<<grid, 64, 0, s>>>(U(a.q), U(a.k), U(a.v_qk), U(a.k_v), U(a.do_qk), a.lse, a.delta, a.lut,
                                          a.counts, a.cap, g, sc_log2, scale, static_cast<bf16*>(dq), map);
    bwd_dkv_kernel<64><<<grid_kv, 256, 0, s>>>(U(a.q), U(a.k), U(a.v_qk), U(a.do_qk), a.lse,
                                            a.delta, a.lut_t, a.counts_t, a.cap_t, g, sc_log2, scale,
                                            static_cast<bf16*>(dk), static_cast<bf16*>(dv));
  }
  return hipGetLastError();
}

}  // namespace sa
