// Per-sequence Top-K budgets (gfx950).
//
// VSA2 ("Improving Video Sparse Attention with Fine-grained Router and Sparse
// Rebasing"), section 1 and its ablation of the TopK scope: one budget for the
// whole sequence (a head), spent where the block probabilities are largest,
// so rows get different counts.  Here the budget is what per-row Top-k would
// keep, T = rows * ceil(k * nblk); the T largest entries of the head's
// row-softmax probabilities win, equal values going to the lower row-major
// index; row i's count c_i is then handed to the selection kernel as a row
// budget, so each row keeps its c_i top-scoring blocks.
//
// The entries are compared through their log-probabilities x_ij = S_ij - L_i
// (L_i the row's log-sum-exp, float64), which order exactly as the
// probabilities do.  The T-th largest x of a head is found by an 8-pass radix
// select over the order-preserving 64-bit key of x (8 bits per pass): every
// pass histograms the entries that still share the found prefix -- per
// workgroup in LDS, merged with integer atomics, so the result does not depend
// on scheduling -- and one wave per head picks the digit.  Runs of equal
// digits (the leading bytes of neighbouring entries mostly agree) are counted
// in registers and added to LDS once per run.  Finally every row counts its
// entries above the threshold and equal to it, and one pass per head hands
// the remaining equal entries to the rows in index order.
#include "sa_launch.h"

#include <math.h>

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerGroup = 8;

// Ascending order-preserving key of a double.
__device__ __forceinline__ uint64_t asc_key(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  return (b >> 63) ? ~b : (b | (1ull << 63));
}

__device__ double block_reduce(double v, double* red, bool is_max) {
  // fixed order: wave butterflies, then the 4 wave results in order
  for (int o = 32; o > 0; o >>= 1) {
    const double w = __shfl_xor(v, o, kWave);
    v = is_max ? fmax(v, w) : v + w;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  double r = red[0];
  for (int w = 1; w < kThreads / kWave; ++w) r = is_max ? fmax(r, red[w]) : r + red[w];
  return r;
}

// L_i = max_j S_ij + ln sum_j exp(S_ij - max), one workgroup per row.
__global__ __launch_bounds__(kThreads) void row_lse_kernel(const double* __restrict__ scores, int n,
                                                           double* __restrict__ lse) {
  __shared__ double red[kThreads / kWave];
  const long long row = blockIdx.x;
  const double* s = scores + row * (long long)n;
  double mx = -INFINITY;
  for (int j = threadIdx.x; j < n; j += kThreads) mx = fmax(mx, s[j]);
  mx = block_reduce(mx, red, true);
  double z = 0.0;
  for (int j = threadIdx.x; j < n; j += kThreads) z += exp(s[j] - mx);
  z = block_reduce(z, red, false);
  if (threadIdx.x == 0) lse[row] = mx + log(z);
}

// state[2 h] = key prefix found so far, state[2 h + 1] = entries still to take
__global__ __launch_bounds__(kThreads) void radix_init_kernel(unsigned long long* __restrict__ state,
                                                              uint32_t* __restrict__ hist, long long total) {
  const int h = blockIdx.x;
  hist[h * 256 + threadIdx.x] = 0u;
  if (threadIdx.x == 0) {
    state[2 * h] = 0ull;
    state[2 * h + 1] = (unsigned long long)total;
  }
}

__global__ __launch_bounds__(kThreads) void radix_hist_kernel(const double* __restrict__ scores,
                                                              const double* __restrict__ lse, int n, int rows,
                                                              const unsigned long long* __restrict__ state,
                                                              uint32_t* __restrict__ hist, int shift) {
  __shared__ uint32_t h[256];
  h[threadIdx.x] = 0u;
  __syncthreads();
  const long long head = blockIdx.y;
  const int r0 = blockIdx.x * kRowsPerGroup;
  const int r1 = min(r0 + kRowsPerGroup, rows);
  const uint64_t prefix = state[2 * head];
  const uint64_t hi = shift >= 56 ? 0ull : (~0ull << (shift + 8));   // bits already decided
  int run_d = -1;
  uint32_t run_c = 0;
  for (int r = r0; r < r1; ++r) {
    const long long row = head * rows + r;
    const double l = lse[row];
    const double* s = scores + row * (long long)n;
    for (int j = threadIdx.x; j < n; j += kThreads) {
      const uint64_t key = asc_key(s[j] - l);
      if ((key & hi) == (prefix & hi)) {
        const int d = (int)((key >> shift) & 255ull);
        if (d != run_d) {
          if (run_c) atomicAdd(&h[run_d], run_c);
          run_d = d;
          run_c = 0;
        }
        ++run_c;
      }
    }
  }
  if (run_c) atomicAdd(&h[run_d], run_c);
  __syncthreads();
  if (h[threadIdx.x]) atomicAdd(&hist[head * 256 + threadIdx.x], h[threadIdx.x]);
}

// The digit holding the remaining rank, counted from the largest keys down.
__global__ __launch_bounds__(kThreads) void radix_pick_kernel(unsigned long long* __restrict__ state,
                                                              uint32_t* __restrict__ hist, int shift) {
  const int h = blockIdx.x;
  __shared__ uint32_t bins[256];
  bins[threadIdx.x] = hist[h * 256 + threadIdx.x];
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long rem = state[2 * h + 1];
    unsigned long long above = 0;
    int d = 255;
    for (; d > 0; --d) {
      if (above + bins[d] >= rem) break;
      above += bins[d];
    }
    state[2 * h] |= (unsigned long long)d << shift;
    state[2 * h + 1] = rem - above;
  }
  hist[h * 256 + threadIdx.x] = 0u;   // cleared for the next pass
}

// Per row: entries above the threshold key and equal to it.
__global__ __launch_bounds__(kThreads) void row_split_kernel(const double* __restrict__ scores,
                                                             const double* __restrict__ lse, int n, int rows,
                                                             const unsigned long long* __restrict__ state,
                                                             int32_t* __restrict__ gt, int32_t* __restrict__ eq) {
  __shared__ int red[2][kThreads / kWave];
  const long long row = blockIdx.x;
  const long long head = row / rows;
  const uint64_t t = state[2 * head];
  const double l = lse[row];
  const double* s = scores + row * (long long)n;
  int a = 0, e = 0;
  for (int j = threadIdx.x; j < n; j += kThreads) {
    const uint64_t key = asc_key(s[j] - l);
    a += key > t;
    e += key == t;
  }
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o, kWave);
    e += __shfl_xor(e, o, kWave);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = a;
    red[1][threadIdx.x >> 6] = e;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int sa = 0, se = 0;
    for (int w = 0; w < kThreads / kWave; ++w) {
      sa += red[0][w];
      se += red[1][w];
    }
    gt[row] = sa;
    eq[row] = se;
  }
}

// Counts: the entries above the threshold, plus the equal ones still owed,
// handed out in row order.  total <= 0 keeps nothing; total >= rows * n keeps all.
__global__ __launch_bounds__(64) void row_budget_kernel(const int32_t* __restrict__ gt,
                                                        const int32_t* __restrict__ eq,
                                                        const unsigned long long* __restrict__ state, int n,
                                                        int rows, long long total, int32_t* __restrict__ budget) {
  const long long head = blockIdx.x;
  if (threadIdx.x != 0) return;
  const bool none = total <= 0, all = total >= (long long)rows * n;
  long long owed = (long long)state[2 * head + 1];
  for (int r = 0; r < rows; ++r) {
    const long long row = head * rows + r;
    int c;
    if (none) {
      c = 0;
    } else if (all) {
      c = n;
    } else {
      const long long take = owed < eq[row] ? (owed > 0 ? owed : 0) : eq[row];
      owed -= take;
      c = gt[row] + (int)take;
    }
    budget[row] = c;
  }
}

}  // namespace

size_t sequence_workspace_bytes(const Geom& g) {
  const size_t rows = (size_t)g.batch * g.heads * g.nblk;
  const size_t heads = (size_t)g.batch * g.heads;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return up(rows * sizeof(double)) + up(heads * 2 * sizeof(unsigned long long)) +
         up(heads * 256 * sizeof(uint32_t)) + 3 * up(rows * sizeof(int32_t));
}

hipError_t launch_sequence_budget(const double* scores, const Geom& g, long long total, void* workspace,
                                  int32_t** budget_out, hipStream_t s) {
  const int n = g.nblk, rows = g.nblk;
  const int heads = g.batch * g.heads;
  const size_t nrows = (size_t)heads * rows;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* w = static_cast<char*>(workspace);
  double* lse = reinterpret_cast<double*>(w);
  w += up(nrows * sizeof(double));
  unsigned long long* state = reinterpret_cast<unsigned long long*>(w);
  w += up((size_t)heads * 2 * sizeof(unsigned long long));
  uint32_t* hist = reinterpret_cast<uint32_t*>(w);
  w += up((size_t)heads * 256 * sizeof(uint32_t));
  int32_t* gt = reinterpret_cast<int32_t*>(w);
  w += up(nrows * sizeof(int32_t));
  int32_t* eq = reinterpret_cast<int32_t*>(w);
  w += up(nrows * sizeof(int32_t));
  int32_t* budget = reinterpret_cast<int32_t*>(w);
  *budget_out = budget;
  row_lse_kernel<<<(unsigned)nrows, kThreads, 0, s>>>(scores, n, lse);
  radix_init_kernel<<<heads, kThreads, 0, s>>>(state, hist, total);
  const dim3 hgrid((rows + kRowsPerGroup - 1) / kRowsPerGroup, heads);
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    radix_hist_kernel<<<hgrid, kThreads, 0, s>>>(scores, lse, n, rows, state, hist, shift);
    radix_pick_kernel<<<heads, kThreads, 0, s>>>(state, hist, shift);
  }
  row_split_kernel<<<(unsigned)nrows, kThreads, 0, s>>>(scores, lse, n, rows, state, gt, eq);
  row_budget_kernel<<<heads, 64, 0, s>>>(gt, eq, state, n, rows, total, budget);
  return hipGetLastError();
}

}  // namespace sa
