// Element order inside one cube-major block of 64 tokens x d dims.
//
// The forward kernel feeds K and V to v_mfma_f32_32x32x16_bf16 straight from
// global memory.  Each operand load is one 16-byte chunk per lane, and a wave's
// 64 chunks must form one contiguous, aligned kilobyte to run at full L2
// bandwidth; natural row-major blocks would give 32-byte pieces of 32 rows.
// So blocks are stored as a sequence of 1 KB "operand chunks":
//
//   QK layout (queries and keys; contraction over d):
//     chunk (t32, ds) = tokens 32*t32 .. +31, dims 16*ds .. +15;
//     chunk index t32*(d/16) + ds; inside it, position p = h*32 + r holds the
//     8 dims 16*ds + 8*h .. +7 of token 32*t32 + r.
//   V layout (values; contraction over tokens):
//     chunk (dt, ks) = dims 32*dt .. +31, tokens 16*ks .. +15;
//     chunk index dt*4 + ks; position p = h*32 + r holds tokens
//     16*ks + 8*h .. +7 of dim 32*dt + r.
//
// Both are permutations of the block's 64*d elements, so a block still
// occupies exactly 64*d contiguous elements at offset block*64*d.
#pragma once

namespace sa {

// Element offset of (slot s, dim c) inside a QK-layout block.
__host__ __device__ __forceinline__ int qk_offset(int s, int c, int d) {
  return ((s >> 5) * (d >> 4) + (c >> 4)) * 512 + ((c >> 3) & 1) * 256 + (s & 31) * 8 + (c & 7);
}

// Element offset of (slot s, dim c) inside a V-layout block.
__host__ __device__ __forceinline__ int v_offset(int s, int c, int d) {
  (void)d;
  return ((c >> 5) * 4 + (s >> 4)) * 512 + ((s >> 3) & 1) * 256 + (c & 31) * 8 + (s & 7);
}

}  // namespace sa
