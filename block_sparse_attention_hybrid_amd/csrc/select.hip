// Hybrid Top-k U Top-p block selection (gfx950): one wavefront per query block
// for rows of up to 1536 blocks, one workgroup of four per longer row.
//
// SpargeAttention2 summary page, "The Hybrid Top-k+Top-p Masking Rule" (Eq. 9):
// a row keeps the union of its Top-k blocks (ceil(k * Tn) largest scores) and
// its Top-p blocks (the shortest prefix of the descending order whose
// cumulative softmax probability reaches p).  Both are prefixes of the same
// order -- score descending, lower block id first on equal scores -- so the
// union is the prefix of length max(kc, pc).  VSA summary page, "Kernel
// Implementation": the result is written as a contiguous list of block ids.
//
// The kernel never sorts the row.  It searches for the boundary of that
// prefix: the set of elements still in question ("members") is split into 256
// buckets that are monotone in the order (linear in the score for the first
// two rounds, then by the next 8 differing bits of the order-preserving
// 64-bit key), a histogram of counts and masses picks the first bucket at
// which both conditions (count >= kc, mass >= p * Z) hold, the buckets before
// it join the kept set, and the search continues inside that bucket.  Once at
// most 64 members are left (usually after the first round) they are copied to
// LDS in ascending id, and each lane takes the exact rank of one member in the
// order and the mass of the members up to it by one pass over that short
// list; the first rank at which both conditions hold closes the prefix.  Only
// a group of more than 64 equal scores is resolved by count instead: its
// members all carry the same mass, so the number taken (in ascending id) is a
// division.  Every round strictly shrinks the member set and the key rounds
// consume 8 key bits each, so the loop ends after at most 10 rounds.
//
// Work split (rows above 1536 blocks; shorter rows use the one-wave kernel
// further below, which runs the same steps): the row's n scores are spread
// over the 4 waves of the workgroup, wave w holding the contiguous ids
// [64 E w, 64 E (w + 1)) as E registers per lane, so every wave compacts its
// own kept ids in ascending order with ballots and only per-wave totals cross
// waves (through LDS).  The histogram is shared; wave 0 scans it and posts
// each round's decision in LDS.
//
// Probabilities are exp2 of the float64 score differences in float32, summed
// as 2^-40 fixed-point integers: integer LDS atomics make the histograms (and
// so the lists) independent of thread scheduling.  Only the scores are kept
// in registers; a probability is taken again wherever it is used, which
// leaves room for one more wave per SIMD.  For rows of up to 2048
// blocks a bucket's count and mass share one 64-bit word (count above bit
// 52), so each element costs one LDS atomic.
#include "sa_launch.h"

#include <math.h>

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr double kFixOne = 1099511627776.0;  // 2^40: fixed-point unit of probability mass
constexpr double kLog2e = 1.4426950408889634;
constexpr int kMaxRounds = 16;
constexpr int kCountShift = 52;              // packed histogram word: count << 52 | mass
constexpr uint64_t kMassMask = (1ull << kCountShift) - 1;
#ifndef SA_SELECT_ONE_WAVE
#define SA_SELECT_ONE_WAVE 1
#endif

// floor(e 2^40 + 0.5) for a probability 0 <= e <= 1, held in the low bits of
// a double: e 2^40 + 0.5 is exact in float64 for every e that does not round
// it below 1 (e has 24 significant bits), and for an integer m < 2^52 the
// double 2^52 + m has exponent field 0x433 and mantissa field m.  Five vector
// operations instead of a general float64 -> uint64 conversion.
__device__ __forceinline__ uint64_t fixed_in_double(float e) {
  const double m = floor(fma((double)e, kFixOne, 0.5));
  return (uint64_t)__double_as_longlong(m + 4503599627370496.0);
}

// the 2^-40 fixed-point mass of probability e
__device__ __forceinline__ uint64_t to_fixed(float e) { return fixed_in_double(e) ^ (0x433ull << 52); }

// one packed histogram word: count 1 (bit kCountShift) and the mass of e
static_assert(kCountShift == 52, "the packed word shares the double's exponent position");
__device__ __forceinline__ uint64_t count_and_mass(float e) { return fixed_in_double(e) ^ (0x432ull << 52); }

__device__ __forceinline__ float prob(double s, double mx) {
  return __builtin_amdgcn_exp2f((float)((s - mx) * kLog2e));
}

// Order-preserving key: descending score <-> ascending key.
__device__ __forceinline__ uint64_t desc_key(double s) {
  const uint64_t b = (uint64_t)__double_as_longlong(s);
  const uint64_t asc = (b >> 63) ? ~b : (b | (1ull << 63));
  return ~asc;
}

// An opaque copy: per-element work on it is redone where it is used instead of
// being hoisted out of the histogram-pass loop, which would keep a precomputed copy of
// every element in registers.
template <typename T>
__device__ __forceinline__ T fresh(T x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Cross-lane steps on the DPP path (a few cycles each) rather than LDS
// permutes.  Reductions combine within rows of 16 lanes (swap neighbours,
// swap pairs, mirror halves, mirror the row), then take the four row results
// with readlane, so the result is wave-uniform.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppRowShr = 0x110;     // + n: row_shr:n (lanes below n read 0)

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, 0xF, 0xF, true);
}

template <int kCtrl>
__device__ __forceinline__ uint64_t dpp64(uint64_t x) {
  return (uint64_t)dpp<kCtrl>((uint32_t)x) | ((uint64_t)dpp<kCtrl>((uint32_t)(x >> 32)) << 32);
}

template <int kCtrl>
__device__ __forceinline__ double dpp_d(double x) {
  return __longlong_as_double((long long)dpp64<kCtrl>((uint64_t)__double_as_longlong(x)));
}

__device__ __forceinline__ uint32_t readlane(uint32_t x, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, l);
}

__device__ __forceinline__ uint64_t readlane64(uint64_t x, int l) {
  return (uint64_t)readlane((uint32_t)x, l) | ((uint64_t)readlane((uint32_t)(x >> 32), l) << 32);
}

__device__ __forceinline__ double readlane_d(double x, int l) {
  return __longlong_as_double((long long)readlane64((uint64_t)__double_as_longlong(x), l));
}

template <typename T, typename Op>
__device__ __forceinline__ T row_reduce(T x, Op op) {
  if constexpr (sizeof(T) == 8 && !__is_same(T, double)) {
    x = op(x, (T)dpp64<kDppXor1>(x));
    x = op(x, (T)dpp64<kDppXor2>(x));
    x = op(x, (T)dpp64<kDppHalfMirror>(x));
    x = op(x, (T)dpp64<kDppMirror>(x));
  } else if constexpr (__is_same(T, double)) {
    x = op(x, dpp_d<kDppXor1>(x));
    x = op(x, dpp_d<kDppXor2>(x));
    x = op(x, dpp_d<kDppHalfMirror>(x));
    x = op(x, dpp_d<kDppMirror>(x));
  } else {
    x = op(x, (T)dpp<kDppXor1>((uint32_t)x));
    x = op(x, (T)dpp<kDppXor2>((uint32_t)x));
    x = op(x, (T)dpp<kDppHalfMirror>((uint32_t)x));
    x = op(x, (T)dpp<kDppMirror>((uint32_t)x));
  }
  return x;
}

template <typename T>
__device__ __forceinline__ T lane_read(T x, int l) {
  if constexpr (__is_same(T, double)) return readlane_d(x, l);
  else if constexpr (sizeof(T) == 8) return (T)readlane64((uint64_t)x, l);
  else return (T)readlane((uint32_t)x, l);
}

template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T x, Op op) {
  x = row_reduce(x, op);
  return op(op(lane_read(x, 0), lane_read(x, 16)), op(lane_read(x, 32), lane_read(x, 48)));
}

__device__ __forceinline__ double wmax(double x) {
  return wave_reduce(x, [](double a, double b) { return fmax(a, b); });
}
__device__ __forceinline__ double wmin(double x) {
  return wave_reduce(x, [](double a, double b) { return fmin(a, b); });
}
__device__ __forceinline__ uint64_t wmin_u64(uint64_t x) {
  return wave_reduce(x, [](uint64_t a, uint64_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint64_t wmax_u64(uint64_t x) {
  return wave_reduce(x, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ int wmin_i32(int x) {
  return wave_reduce(x, [](int a, int b) { return a < b ? a : b; });
}

// Inclusive prefix sums over the 64 lanes of a count and a mass: Hillis-Steele
// inside each row of 16, then the totals of the rows before.
__device__ __forceinline__ void wave_scan(uint32_t& c, uint64_t& m, int lane) {
  c += dpp<kDppRowShr + 1>(c);
  m += dpp64<kDppRowShr + 1>(m);
  c += dpp<kDppRowShr + 2>(c);
  m += dpp64<kDppRowShr + 2>(m);
  c += dpp<kDppRowShr + 4>(c);
  m += dpp64<kDppRowShr + 4>(m);
  c += dpp<kDppRowShr + 8>(c);
  m += dpp64<kDppRowShr + 8>(m);
  const uint32_t c0 = readlane(c, 15), c1 = readlane(c, 31), c2 = readlane(c, 47);
  const uint64_t m0 = readlane64(m, 15), m1 = readlane64(m, 31), m2 = readlane64(m, 47);
  const int row = lane >> 4;
  c += row == 0 ? 0u : row == 1 ? c0 : row == 2 ? c0 + c1 : c0 + c1 + c2;
  m += row == 0 ? 0ull : row == 1 ? m0 : row == 2 ? m0 + m1 : m0 + m1 + m2;
}

template <typename T, int E>
__global__ __launch_bounds__(kThreads) void select_kernel(const T* __restrict__ scores, int n,
                                                          int kc_default, double p,
                                                          const int32_t* __restrict__ row_budget,
                                                          int32_t* __restrict__ lut,
                                                          int32_t* __restrict__ counts, int cap) {
  // counts stay below 2^12 and masses below 2^52 while n <= 2048
  constexpr bool kPacked = E * kThreads <= 2048;
  __shared__ unsigned long long hist[256];
  __shared__ uint32_t hcnt[kPacked ? 1 : 256];
  __shared__ unsigned long long ckey[kWave], cmass[kWave];
  __shared__ double xlo[kWaves], xhi[kWaves];
  __shared__ unsigned long long xk0[kWaves], xk1[kWaves];
  __shared__ int xn[kWaves];
  __shared__ unsigned long long xdec[5];   // bucket, its count, count and mass before it, target
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int first_id = wave * kWave * E;
  const uint64_t lt = lanemask_lt();
  const long long row = blockIdx.x;
  const T* srow = scores + row * (long long)n;

  // every load first, at clamped in-row addresses, then the masking: no load
  // waits behind a branch
  double s[E];   // float32 scores are widened exactly on load
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = first_id + e * kWave + lane;
    s[e] = srow[j < n ? j : n - 1];
  }

  int kc = row_budget != nullptr ? row_budget[row] : kc_default;
  kc = kc < 0 ? 0 : (kc > n ? n : kc);
  uint32_t valid = 0;   // per-lane element masks: E <= 16 bits
  double mx = -INFINITY, lo0 = INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool in = first_id + e * kWave + lane < n;
    const double v = s[e] == 0.0 ? 0.0 : s[e];  // -0 and +0 are the same score
    s[e] = in ? v : 0.0;
    valid |= (uint32_t)in << e;
    mx = fmax(mx, in ? v : -INFINITY);
    lo0 = fmin(lo0, in ? v : INFINITY);
  }
  mx = wmax(mx);
  lo0 = wmin(lo0);
  if (lane == 0) {
    xhi[wave] = mx;
    xlo[wave] = lo0;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mx = fmax(mx, xhi[w]);
    lo0 = fmin(lo0, xlo[w]);
  }

  const bool keep_all = (p >= 1.0) || (kc >= n);
  const bool keep_none = !keep_all && kc == 0 && !(p > 0.0);
  uint32_t above = 0, member = 0;
  uint64_t kept_rank = 0;    // members kept by rank: bit = member index in ascending id
  long long take = -1;       // >= 0: the first `take` members by id are kept
  int mbase = 0;             // members held by the waves before this one

  if (keep_all) {
    above = valid;
  } else if (!keep_none) {
    member = valid;
    int m = n;                 // members left (uniform over the workgroup)
    long long cnt_above = 0;
    unsigned long long mass_above = 0, target = 0;
    bool equal = false;        // all members share the score eq
    double eq = 0.0;
    for (int round = 0; round < kMaxRounds && (round == 0 || m > kWave); ++round) {
      double lo = lo0, hi = mx;
      if (round > 0) {
        lo = INFINITY;
        hi = -INFINITY;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const bool mem = (member >> e) & 1u;
          lo = fmin(lo, mem ? s[e] : INFINITY);
          hi = fmax(hi, mem ? s[e] : -INFINITY);
        }
        lo = wmin(lo);
        hi = wmax(hi);
        if (lane == 0) {
          xlo[wave] = lo;
          xhi[wave] = hi;
        }
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          lo = fmin(lo, xlo[w]);
          hi = fmax(hi, xhi[w]);
        }
      }
      if (!(lo < hi)) {
        equal = true;
        eq = hi;
        if (round == 0) {  // every score equal: every mass is exp2(0) = 1
          const unsigned long long z = (unsigned long long)n * to_fixed(1.0f);
          target = p > 0.0 ? (unsigned long long)ceil(p * (double)z) : 0ull;
        }
        break;
      }
      // bucket function of this round
      const double w = 256.0 / (hi - lo);
      const bool linear = round < 2 && w < 1e300;
      int shift = 0;
      if (!linear) {
        uint64_t kmin = ~0ull, kmax = 0;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if ((member >> e) & 1u) {
            const uint64_t k = desc_key(fresh(s[e]));
            kmin = k < kmin ? k : kmin;
            kmax = k > kmax ? k : kmax;
          }
        kmin = wmin_u64(kmin);
        kmax = wmax_u64(kmax);
        if (lane == 0) {
          xk0[wave] = kmin;
          xk1[wave] = kmax;
        }
        __syncthreads();
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
          kmin = xk0[v] < kmin ? xk0[v] : kmin;
          kmax = xk1[v] > kmax ? xk1[v] : kmax;
        }
        const int hb = 63 - __clzll((long long)(kmin ^ kmax));
        shift = hb >= 7 ? hb - 7 : 0;
      }
      auto bucket = [&](double v) -> int {
        if (linear) {
          const int b = (int)((hi - v) * w);
          return b > 255 ? 255 : b;
        }
        return (int)((desc_key(v) >> shift) & 255ull);
      };

      // the exchange above (or, in the first histogram pass, the one before the loop) orders
      // the previous pass's histogram reads before this clear
      hist[threadIdx.x] = 0ull;
      if constexpr (!kPacked) hcnt[threadIdx.x] = 0u;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((member >> e) & 1u) {
          const int b = bucket(fresh(s[e]));
          const unsigned long long f = to_fixed(prob(fresh(s[e]), mx));
          if constexpr (kPacked) {
            atomicAdd(&hist[b], (1ull << kCountShift) | f);
          } else {
            atomicAdd(&hcnt[b], 1u);
            atomicAdd(&hist[b], f);
          }
        }
      __syncthreads();

      // wave 0 scans the 256 buckets (lane L taking buckets 4L .. 4L+3) and
      // posts the decision; the other waves read it after the barrier
      if (wave == 0) {
        uint32_t c4[4];
        unsigned long long m4[4];
        uint32_t lc = 0;
        unsigned long long lm = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const unsigned long long hw = hist[lane * 4 + t];
          if constexpr (kPacked) {
            c4[t] = (uint32_t)(hw >> kCountShift);
            m4[t] = hw & kMassMask;
          } else {
            c4[t] = hcnt[lane * 4 + t];
            m4[t] = hw;
          }
          lc += c4[t];
          lm += m4[t];
        }
        uint32_t ic = lc;
        uint64_t im = lm;
        wave_scan(ic, im, lane);
        if (round == 0) {  // every element is a member: the total is Z
          const unsigned long long z = readlane64(im, kWave - 1);
          target = p > 0.0 ? (unsigned long long)ceil(p * (double)z) : 0ull;
        }
        uint32_t xc = ic - lc;            // exclusive prefix of this lane's first bucket
        unsigned long long xm = im - lm;
        int first = 4;
        uint32_t first_xc = 0, first_c = 0;
        unsigned long long first_xm = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bool ok = (cnt_above + (long long)(xc + c4[t]) >= kc) && (mass_above + xm + m4[t] >= target);
          if (ok && first == 4) {
            first = t;
            first_xc = xc;
            first_xm = xm;
            first_c = c4[t];
          }
          xc += c4[t];
          xm += m4[t];
        }
        const uint64_t hit = ballot(first < 4);
        const int src = hit ? (__ffsll((long long)hit) - 1) : (kWave - 1);
        if (!hit && lane == kWave - 1) {  // unreachable: all members always satisfy both
          first = 3;
          first_xc = ic - c4[3];
          first_xm = im - m4[3];
          first_c = c4[3];
        }
        if (lane == 0) {
          xdec[0] = (unsigned long long)(4 * src + (int)readlane((uint32_t)first, src));
          xdec[1] = readlane(first_c, src);
          xdec[2] = readlane(first_xc, src);
          xdec[3] = readlane64(first_xm, src);
          xdec[4] = target;
        }
      }
      __syncthreads();
      const int bstar = (int)xdec[0];
      m = (int)xdec[1];
      cnt_above += (long long)xdec[2];
      mass_above += xdec[3];
      target = xdec[4];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool mem = (member >> e) & 1u;
        const int b = bucket(fresh(s[e]));
        above |= (uint32_t)(mem && b < bstar) << e;
        member &= ~((uint32_t)(mem && b != bstar) << e);
      }
    }

    // members of the waves before this one (ascending id across the row)
    int nm = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) nm += __popcll(ballot((member >> e) & 1u));
    if (lane == 0) xn[wave] = nm;
    __syncthreads();
    for (int v = 0; v < wave; ++v) mbase += xn[v];

    if (m <= kWave) {
      // exact finish: members to LDS in ascending id, then rank by one pass
      int seen = mbase;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool is_mem = (member >> e) & 1u;
        const uint64_t bm = ballot(is_mem);
        if (bm) {
          if (is_mem) {
            const int idx = seen + __popcll(bm & lt);
            ckey[idx] = desc_key(s[e]);
            cmass[idx] = to_fixed(prob(s[e], mx));
          }
          seen += __popcll(bm);
        }
      }
      __syncthreads();
      // every wave ranks the same list, so all hold the same decision
      const bool mine = lane < m;
      const unsigned long long kk = mine ? ckey[lane] : ~0ull;
      int r = 0;                      // members ahead of this one in the order
      unsigned long long pm = 0;      // mass of the members up to and including it
      for (int j = 0; j < m; ++j) {
        const unsigned long long kj = ckey[j];
        const bool ahead = kj < kk || (kj == kk && j < lane);
        r += ahead ? 1 : 0;
        pm += (ahead || j == lane) ? cmass[j] : 0ull;
      }
      const bool ok = mine && (cnt_above + r + 1 >= kc) && (mass_above + pm >= target);
      const int rstar = wmin_i32(ok ? r : kWave);
      kept_rank = ballot(mine && r <= rstar);
    } else {
      // more than 64 members of one score (the pass limit is never reached):
      // equal masses u, so the count taken is a division
      (void)equal;
      const unsigned long long u = to_fixed(prob(eq, mx));
      long long need = kc - cnt_above;
      if (mass_above < target && u > 0) {
        const long long need_p = (long long)((target - mass_above + u - 1) / u);
        need = need_p > need ? need_p : need;
      }
      take = need < 0 ? 0 : (need > (long long)m ? (long long)m : need);
    }
  }

  // ascending-id compaction: kept = above U (selected members); this wave's
  // ids follow those kept by the waves before it
  uint64_t bk[E];
  int nk = 0;
  if (ballot(member != 0u) == 0ull) {
    // no members in this wave (the common case): kept = above
#pragma unroll
    for (int e = 0; e < E; ++e) {
      bk[e] = ballot((above >> e) & 1u);
      nk += __popcll(bk[e]);
    }
  } else {
    int seen = mbase;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool is_mem = (member >> e) & 1u;
      const uint64_t bm = ballot(is_mem);
      const int rank = seen + __popcll(bm & lt);
      seen += __popcll(bm);
      const bool sel = take >= 0 ? rank < take : (rank < kWave && ((kept_rank >> rank) & 1ull));
      bk[e] = ballot(((above >> e) & 1u) || (is_mem && sel));
      nk += __popcll(bk[e]);
    }
  }
  __syncthreads();  // the member counts have been read before they are overwritten
  if (lane == 0) xn[wave] = nk;
  __syncthreads();
  int written = 0, total = 0;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    written += v < wave ? xn[v] : 0;
    total += xn[v];
  }
  int32_t* out = lut + row * (long long)cap;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool keep = (bk[e] >> lane) & 1ull;
    const int pos = written + __popcll(bk[e] & lt);
    written += __popcll(bk[e]);
    if (keep && pos < cap) out[pos] = first_id + e * kWave + lane;
  }
  if (threadIdx.x == 0) counts[row] = (int32_t)total;
}

template <int E, typename T>
hipError_t launch_e(const T* scores, const Geom& g, int kc, double p, const int32_t* rb,
                    int32_t* lut, int32_t* counts, int cap, hipStream_t s, int rows_per_head) {
  const long long rows = (long long)g.batch * g.heads * rows_per_head;
  if (rows == 0) return hipSuccess;
  select_kernel<T, E><<<dim3((unsigned)rows), kThreads, 0, s>>>(scores, g.nblk, kc, p, rb, lut, counts, cap);
  return hipGetLastError();
}

// One wavefront per row, for rows of up to 1536 blocks (E <= 24 registers per
// lane).  The same selection as select_kernel -- the same bucket functions,
// fixed-point masses, decisions and exact finish, so the same lists -- with
// the row held by a single wave: the reductions, the histogram scan and the
// decision of every round are done once per row instead of by four waves
// that then exchange them through LDS behind barriers.  A workgroup holds
// four independent rows, each wave with its own LDS histogram and member
// list; no barrier is needed (a wave's LDS operations are ordered, and the
// wavefront fences below keep the compiler from moving reads of other
// lanes' buckets across the atomics).
//
// The kernel is bound by latency more than by issue, so it is held to 128
// registers (four waves per SIMD): the scores stay in registers, and each
// element's probability is taken again where it is used (the histogram
// passes and the exact finish) instead of being kept beside its score.  At
// 1,440 blocks per row this runs 15% faster than the 167-register form at
// three waves per SIMD, with the same lists.
constexpr int kRowsPerSelectGroup = 4;

__device__ __forceinline__ void wave_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

template <typename T, int E>
__global__ __launch_bounds__(kWave * kRowsPerSelectGroup) __attribute__((amdgpu_waves_per_eu(4)))
void select_wave_kernel(
    const T* __restrict__ scores, int n, int kc_default, double p, const int32_t* __restrict__ row_budget,
    int32_t* __restrict__ lut, int32_t* __restrict__ counts, int cap, long long rows) {
  static_assert(E * kWave <= 2048, "packed histogram words need n <= 2048");
  __shared__ unsigned long long hist_all[kRowsPerSelectGroup][256];
  __shared__ unsigned long long ckey_all[kRowsPerSelectGroup][kWave], cmass_all[kRowsPerSelectGroup][kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * kRowsPerSelectGroup + wave;
  if (row >= rows) return;   // no barrier below: a wave past the rows just leaves
  unsigned long long* hist = hist_all[wave];
  unsigned long long* ckey = ckey_all[wave];
  unsigned long long* cmass = cmass_all[wave];
  const uint64_t lt = lanemask_lt();
  const T* srow = scores + row * (long long)n;

  // every load first, at clamped in-row addresses, then the masking
  double s[E];   // float32 scores are widened exactly on load
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = e * kWave + lane;
    s[e] = srow[j < n ? j : n - 1];
  }
  int kc = row_budget != nullptr ? row_budget[row] : kc_default;
  kc = kc < 0 ? 0 : (kc > n ? n : kc);
  uint32_t valid = 0;
  double mx = -INFINITY, lo0 = INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool in = e * kWave + lane < n;
    const double v = s[e] == 0.0 ? 0.0 : s[e];  // -0 and +0 are the same score
    s[e] = in ? v : 0.0;
    valid |= (uint32_t)in << e;
    mx = fmax(mx, in ? v : -INFINITY);
    lo0 = fmin(lo0, in ? v : INFINITY);
  }
  mx = wmax(mx);
  lo0 = wmin(lo0);

  const bool keep_all = (p >= 1.0) || (kc >= n);
  const bool keep_none = !keep_all && kc == 0 && !(p > 0.0);
  uint32_t above = 0, member = 0;
  uint64_t kept_rank = 0;    // members kept by rank: bit = member index in ascending id
  long long take = -1;       // >= 0: the first `take` members by id are kept

  if (keep_all) {
    above = valid;
  } else if (!keep_none) {
    member = valid;
    int m = n;                 // members left
    long long cnt_above = 0;
    unsigned long long mass_above = 0, target = 0;
    double eq = 0.0;
    for (int round = 0; round < kMaxRounds && (round == 0 || m > kWave); ++round) {
      double lo = lo0, hi = mx;
      if (round > 0) {
        lo = INFINITY;
        hi = -INFINITY;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const bool mem = (member >> e) & 1u;
          lo = fmin(lo, mem ? s[e] : INFINITY);
          hi = fmax(hi, mem ? s[e] : -INFINITY);
        }
        lo = wmin(lo);
        hi = wmax(hi);
      }
      if (!(lo < hi)) {
        eq = hi;
        if (round == 0) {  // every score equal: every mass is exp2(0) = 1
          const unsigned long long z = (unsigned long long)n * to_fixed(1.0f);
          target = p > 0.0 ? (unsigned long long)ceil(p * (double)z) : 0ull;
        }
        break;
      }
      // bucket function of this round
      const double w = 256.0 / (hi - lo);
      const bool linear = round < 2 && w < 1e300;
      int shift = 0;
      if (!linear) {
        uint64_t kmin = ~0ull, kmax = 0;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if ((member >> e) & 1u) {
            const uint64_t k = desc_key(fresh(s[e]));
            kmin = k < kmin ? k : kmin;
            kmax = k > kmax ? k : kmax;
          }
        kmin = wmin_u64(kmin);
        kmax = wmax_u64(kmax);
        const int hb = 63 - __clzll((long long)(kmin ^ kmax));
        shift = hb >= 7 ? hb - 7 : 0;
      }
      auto bucket = [&](double v) -> int {
        if (linear) {
          const int b = (int)((hi - v) * w);
          return b > 255 ? 255 : b;
        }
        return (int)((desc_key(v) >> shift) & 255ull);
      };

#pragma unroll
      for (int t = 0; t < 4; ++t) hist[lane * 4 + t] = 0ull;
      wave_fence();
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((member >> e) & 1u) {
          const int b = bucket(fresh(s[e]));
          atomicAdd(&hist[b], count_and_mass(prob(fresh(s[e]), mx)));
        }
      wave_fence();

      // lane L takes buckets 4L .. 4L+3; the first bucket at which both
      // conditions hold closes the kept prefix
      uint32_t c4[4];
      unsigned long long m4[4];
      uint32_t lc = 0;
      unsigned long long lm = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const unsigned long long hw = hist[lane * 4 + t];
        c4[t] = (uint32_t)(hw >> kCountShift);
        m4[t] = hw & kMassMask;
        lc += c4[t];
        lm += m4[t];
      }
      uint32_t ic = lc;
      uint64_t im = lm;
      wave_scan(ic, im, lane);
      if (round == 0) {  // every element is a member: the total is Z
        const unsigned long long z = readlane64(im, kWave - 1);
        target = p > 0.0 ? (unsigned long long)ceil(p * (double)z) : 0ull;
      }
      uint32_t xc = ic - lc;
      unsigned long long xm = im - lm;
      int first = 4;
      uint32_t first_xc = 0, first_c = 0;
      unsigned long long first_xm = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bool ok = (cnt_above + (long long)(xc + c4[t]) >= kc) && (mass_above + xm + m4[t] >= target);
        if (ok && first == 4) {
          first = t;
          first_xc = xc;
          first_xm = xm;
          first_c = c4[t];
        }
        xc += c4[t];
        xm += m4[t];
      }
      const uint64_t hit = ballot(first < 4);
      const int src = hit ? (__ffsll((long long)hit) - 1) : (kWave - 1);
      if (!hit && lane == kWave - 1) {  // unreachable: all members always satisfy both
        first = 3;
        first_xc = ic - c4[3];
        first_xm = im - m4[3];
        first_c = c4[3];
      }
      const int bstar = 4 * src + (int)readlane((uint32_t)first, src);
      m = (int)readlane(first_c, src);
      cnt_above += (long long)readlane(first_xc, src);
      mass_above += readlane64(first_xm, src);
      wave_fence();   // the histogram reads are done before the next round clears it
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool mem = (member >> e) & 1u;
        const int b = bucket(fresh(s[e]));
        above |= (uint32_t)(mem && b < bstar) << e;
        member &= ~((uint32_t)(mem && b != bstar) << e);
      }
    }

    if (m <= kWave) {
      // exact finish: members to LDS in ascending id, then rank by one pass
      int seen = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool is_mem = (member >> e) & 1u;
        const uint64_t bm = ballot(is_mem);
        if (bm) {
          if (is_mem) {
            const int idx = seen + __popcll(bm & lt);
            ckey[idx] = desc_key(s[e]);
            cmass[idx] = to_fixed(prob(s[e], mx));
          }
          seen += __popcll(bm);
        }
      }
      wave_fence();
      const bool mine = lane < m;
      const unsigned long long kk = mine ? ckey[lane] : ~0ull;
      int r = 0;                      // members ahead of this one in the order
      unsigned long long pm = 0;      // mass of the members up to and including it
      for (int j = 0; j < m; ++j) {
        const unsigned long long kj = ckey[j];
        const bool ahead = kj < kk || (kj == kk && j < lane);
        r += ahead ? 1 : 0;
        pm += (ahead || j == lane) ? cmass[j] : 0ull;
      }
      const bool ok = mine && (cnt_above + r + 1 >= kc) && (mass_above + pm >= target);
      const int rstar = wmin_i32(ok ? r : kWave);
      kept_rank = ballot(mine && r <= rstar);
    } else {
      // more than 64 members of one score: equal masses u, so the count taken
      // is a division
      const unsigned long long u = to_fixed(prob(eq, mx));
      long long need = kc - cnt_above;
      if (mass_above < target && u > 0) {
        const long long need_p = (long long)((target - mass_above + u - 1) / u);
        need = need_p > need ? need_p : need;
      }
      take = need < 0 ? 0 : (need > (long long)m ? (long long)m : need);
    }
  }

  // ascending-id compaction: kept = above U (selected members)
  int32_t* out = lut + row * (long long)cap;
  int written = 0, seen = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool is_mem = (member >> e) & 1u;
    const uint64_t bm = ballot(is_mem);
    const int rank = seen + __popcll(bm & lt);
    seen += __popcll(bm);
    const bool sel = take >= 0 ? rank < take : (rank < kWave && ((kept_rank >> rank) & 1ull));
    const bool keep = ((above >> e) & 1u) || (is_mem && sel);
    const uint64_t bk = ballot(keep);
    const int pos = written + __popcll(bk & lt);
    written += __popcll(bk);
    if (keep && pos < cap) out[pos] = e * kWave + lane;
  }
  if (lane == 0) counts[row] = (int32_t)written;
}

template <int E, typename T>
hipError_t launch_wave_e(const T* scores, const Geom& g, int kc, double p, const int32_t* rb,
                         int32_t* lut, int32_t* counts, int cap, hipStream_t s, int rows_per_head) {
  const long long rows = (long long)g.batch * g.heads * rows_per_head;
  if (rows == 0) return hipSuccess;
  const long long grid = (rows + kRowsPerSelectGroup - 1) / kRowsPerSelectGroup;
  select_wave_kernel<T, E><<<dim3((unsigned)grid), kWave * kRowsPerSelectGroup, 0, s>>>(scores, g.nblk, kc, p, rb,
                                                                                    lut, counts, cap, rows);
  return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t select_t(const T* scores, const Geom& g, int kc_default, double p,
                    const int32_t* row_budget, int32_t* lut, int32_t* counts, int cap, hipStream_t s,
                    int rows_per_head) {
  const int n = g.nblk;  // at most 4096 (checked by the caller)
  if (rows_per_head < 0) rows_per_head = n;
#if SA_SELECT_ONE_WAVE
  // rows of up to 1536 blocks: one wavefront per row
  if (n <= 64) return launch_wave_e<1>(scores, g, kc_default, p, row_budget, lut, counts, cap, s, rows_per_head);
  if (n <= 256) return launch_wave_e<4>(scores, g, kc_default, p, row_budget, lut, counts, cap, s, rows_per_head);
  if (n <= 512) return launch_wave_e<8>(scores, g, kc_default, p, row_budget, lut, counts, cap, s, rows_per_head);
  if (n <= 768) return launch_wave_e<12>(scores, g, kc_default, p, row_budget, lut, counts, cap, s, rows_per_head);
  if (n <= 1024) return launch_wave_e<16>(scores, g, kc_default, p, row_budget, lut, counts, cap, s, rows_per_head);
  if (n <= 1536) return launch_wave_e<24>(scores, g, kc_default, p, row_budget, lut, counts, cap, s, rows_per_head);
#endif
  if (n <= 256) return launch_e<1>(scores, g, kc_default, p, row_budget, lut, counts, cap, s, rows_per_head);
  if (n <= 512) return launch_e<2>(scores, g, kc_default, p, row_budget, lut, counts, cap, s, rows_per_head);
  if (n <= 1024) return launch_e<4>(scores, g, kc_default, p, row_budget, lut, counts, cap, s, rows_per_head);
  if (n <= 1536) return launch_e<6>(scores, g, kc_default, p, row_budget, lut, counts, cap, s, rows_per_head);
  if (n <= 2048) return launch_e<8>(scores, g, kc_default, p, row_budget, lut, counts, cap, s, rows_per_head);
  if (n <= 3072) return launch_e<12>(scores, g, kc_default, p, row_budget, lut, counts, cap, s, rows_per_head);
  return launch_e<16>(scores, g, kc_default, p, row_budget, lut, counts, cap, s, rows_per_head);
}

hipError_t launch_select(const double* scores, const Geom& g, int kc_default, double p,
                         const int32_t* row_budget, int32_t* lut, int32_t* counts, int cap,
                         hipStream_t s, int rows_per_head) {
  return select_t(scores, g, kc_default, p, row_budget, lut, counts, cap, s, rows_per_head);
}

hipError_t launch_select(const float* scores, const Geom& g, int kc_default, double p,
                         const int32_t* row_budget, int32_t* lut, int32_t* counts, int cap,
                         hipStream_t s, int rows_per_head) {
  return select_t(scores, g, kc_default, p, row_budget, lut, counts, cap, s, rows_per_head);
}

}  // namespace sa
