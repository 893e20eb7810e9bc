// XCD-aware mapping of a 1-D grid of workgroups to rows (gfx950).
//
// Workgroups are dispatched round-robin over the 8 XCDs (XCD = workgroup id
// mod 8), and each XCD has its own L2.  Rows here are (batch*head, block)
// pairs walked in order; neighbouring blocks of one head have overlapping
// kept lists, so an XCD that sweeps a contiguous run of one head's blocks
// finds more of their K/V (or Q/dO) tiles in its L2.
#pragma once

#include <hip/hip_runtime.h>

namespace sa {

constexpr int kXcds = 8;

#ifndef SA_XCD_GROUP
#define SA_XCD_GROUP 4
#endif
// Workgroups are dispatched round-robin over the 8 XCDs (XCD = w % 8).  The
// XCDs form 8/G groups of G; group `grp` takes the contiguous row range
// [grp*range, (grp+1)*range).  The range is cut into chunks of c = nblk/G
// blocks (one G-th of a head) dealt round-robin to the G XCDs of the group,
// each XCD sweeping its chunks in order: G XCDs work on the same head at
// once, each on neighbouring blocks.
struct RowMap {
  int rows;     // batch * heads * nblk
  int range;    // rows per XCD group
  int chunk;    // rows per chunk
  int per_xcd;  // workgroups per XCD
};

template <int G = SA_XCD_GROUP>
__host__ __device__ inline RowMap make_rowmap(int nblk, int heads_total) {
  static_assert(G >= 1 && G <= kXcds && kXcds % G == 0, "XCD group must divide 8");
  RowMap m;
  m.rows = nblk * heads_total;
  const int ranges = kXcds / G;
  m.range = (m.rows + ranges - 1) / ranges;
  m.chunk = (nblk + G - 1) / G;
  const int chunks = (m.range + m.chunk - 1) / m.chunk;
  m.per_xcd = (chunks + G - 1) / G * m.chunk;
  return m;
}

// Row of workgroup w, or -1 if w has no row (G as in make_rowmap).
template <int G = SA_XCD_GROUP>
__device__ __forceinline__ int row_of_workgroup(int w, const RowMap& m) {
  const int x = w % kXcds, k = w / kXcds;
  const int grp = x / G, sub = x % G;
  const int q = k / m.chunk, o = k - q * m.chunk;
  const long long in_range = ((long long)q * G + sub) * m.chunk + o;
  const long long row = (long long)grp * m.range + in_range;
  if (in_range >= m.range || row >= m.rows) return -1;
  return (int)row;
}

}  // namespace sa
