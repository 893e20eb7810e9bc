// Device-side helpers shared by the gfx950 kernels of the sparse-attention
// library: geometry of cube-major tensors, bf16 vector types, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kBlock = 64;   // tokens per cube / block
constexpr int kWave = 64;    // CDNA wavefront width

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(double)))) double f64x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

// Geometry of one call, by value in every kernel's arguments.
struct Geom {
  int batch, heads, frames, height, width, d;
  int ct, ch, cw;        // cube sides, ct*ch*cw == 64
  int nt, nh, nw, nblk;  // cubes per side and in total
  long long n_real, n_pad;
};

// Cube coordinates of block i.
__device__ __forceinline__ void block_coords(const Geom& g, int i, int& bt, int& bh, int& bw) {
  bw = i % g.nw;
  const int r = i / g.nw;
  bh = r % g.nh;
  bt = r / g.nh;
}

// Offsets (tt, hh, ww) inside the cube of slot s.
__device__ __forceinline__ void slot_offsets(const Geom& g, int s, int& tt, int& hh, int& ww) {
  ww = s % g.cw;
  const int r = s / g.cw;
  hh = r % g.ch;
  tt = r / g.ch;
}

// Number of real tokens in block i.
__device__ __forceinline__ int block_real_count(const Geom& g, int i) {
  int bt, bh, bw;
  block_coords(g, i, bt, bh, bw);
  const int rt = min(g.ct, g.frames - bt * g.ct);
  const int rh = min(g.ch, g.height - bh * g.ch);
  const int rw = min(g.cw, g.width - bw * g.cw);
  return rt * rh * rw;
}

// Bit s set iff slot s of block i holds a real token.
__device__ __forceinline__ uint64_t block_real_mask(const Geom& g, int i) {
  int bt, bh, bw;
  block_coords(g, i, bt, bh, bw);
  const int rt = min(g.ct, g.frames - bt * g.ct);
  const int rh = min(g.ch, g.height - bh * g.ch);
  const int rw = min(g.cw, g.width - bw * g.cw);
  if (rt == g.ct && rh == g.ch && rw == g.cw) return ~0ull;
  uint64_t m = 0;
  for (int s = 0; s < kBlock; ++s) {
    int tt, hh, ww;
    slot_offsets(g, s, tt, hh, ww);
    if (tt < rt && hh < rh && ww < rw) m |= 1ull << s;
  }
  return m;
}

// The same mask from a whole wavefront at once: lane l passes the offsets of
// slot l (slot_offsets(g, l, ...)), i is wave-uniform and every lane is
// active.  One ballot instead of a loop over the 64 slots.
__device__ __forceinline__ uint64_t block_real_mask_wave(const Geom& g, int i, int lt, int lh, int lw) {
  int bt, bh, bw;
  block_coords(g, i, bt, bh, bw);
  const int rt = min(g.ct, g.frames - bt * g.ct);
  const int rh = min(g.ch, g.height - bh * g.ch);
  const int rw = min(g.cw, g.width - bw * g.cw);
  return __ballot(lt < rt && lh < rh && lw < rw);
}

// Row-major token index of slot s of block i, or -1 for a pad slot.
__device__ __forceinline__ long long slot_token(const Geom& g, int i, int s) {
  int bt, bh, bw, tt, hh, ww;
  block_coords(g, i, bt, bh, bw);
  slot_offsets(g, s, tt, hh, ww);
  const int t = bt * g.ct + tt, h = bh * g.ch + hh, w = bw * g.cw + ww;
  if (t >= g.frames || h >= g.height || w >= g.width) return -1;
  return ((long long)t * g.height + h) * g.width + w;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ double wave_min(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmin(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t w = __shfl_xor(v, o, kWave);
    v = w < v ? w : v;
  }
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

}  // namespace sa
