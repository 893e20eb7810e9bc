// Hybrid Top-k U Top-p block selection, one wavefront per query block (gfx950).
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
// it join the kept set, and the search continues inside that bucket until one
// element or a group of equal scores is left; equal scores are then taken in
// ascending id.  Every round strictly shrinks the member set and the key
// rounds consume 8 key bits each, so the loop ends after at most 10 rounds.
//
// Probabilities are exp2 of the float64 score differences in float32, summed
// as 2^-40 fixed-point integers: integer LDS atomics make the histograms (and
// so the lists) independent of thread scheduling.  Kept ids are compacted in
// ascending order with wave ballots.
#include "sa_launch.h"

#include <math.h>

namespace sa {

namespace {

constexpr double kFixOne = 1099511627776.0;  // 2^40: fixed-point unit of probability mass
constexpr double kLog2e = 1.4426950408889634;
constexpr int kMaxRounds = 16;

__device__ __forceinline__ uint64_t to_fixed(float e) {
  return (uint64_t)((double)e * kFixOne + 0.5);
}

// Order-preserving key: descending score <-> ascending key.
__device__ __forceinline__ uint64_t desc_key(double s) {
  const uint64_t b = (uint64_t)__double_as_longlong(s);
  const uint64_t asc = (b >> 63) ? ~b : (b | (1ull << 63));
  return ~asc;
}

template <int E>
__global__ __launch_bounds__(kWave) void select_kernel(const double* __restrict__ scores, int n,
                                                       int kc_default, double p,
                                                       const int32_t* __restrict__ row_budget,
                                                       int32_t* __restrict__ lut,
                                                       int32_t* __restrict__ counts, int cap) {
  __shared__ uint32_t hcnt[256];
  __shared__ unsigned long long hmass[256];
  const long long row = blockIdx.x;
  const int lane = threadIdx.x;
  const double* srow = scores + row * (long long)n;

  int kc = row_budget != nullptr ? row_budget[row] : kc_default;
  kc = kc < 0 ? 0 : (kc > n ? n : kc);

  double s[E];
  float ev[E];
  uint64_t valid = 0;
  double mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = e * kWave + lane;
    s[e] = 0.0;
    ev[e] = 0.f;
    if (j < n) {
      double v = srow[j];
      if (v == 0.0) v = 0.0;  // -0 and +0 are the same score
      s[e] = v;
      valid |= 1ull << e;
      mx = fmax(mx, v);
    }
  }
  mx = wave_max(mx);

  const bool keep_all = (p >= 1.0) || (kc >= n);
  const bool keep_none = !keep_all && kc == 0 && !(p > 0.0);
  uint64_t above = 0, member = 0;
  long long take = 0;  // members kept, taken in ascending id

  if (keep_all) {
    above = valid;
  } else if (!keep_none) {
    unsigned long long zpart = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((valid >> e) & 1ull) {
        ev[e] = __builtin_amdgcn_exp2f((float)((s[e] - mx) * kLog2e));
        zpart += to_fixed(ev[e]);
      }
    }
    const unsigned long long z = wave_sum(zpart);
    const unsigned long long target = p > 0.0 ? (unsigned long long)ceil(p * (double)z) : 0ull;

    member = valid;
    long long cnt_above = 0;
    unsigned long long mass_above = 0;
    bool ties = false;
    for (int round = 0; round < kMaxRounds; ++round) {
      double lo = INFINITY, hi = -INFINITY;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((member >> e) & 1ull) {
          lo = fmin(lo, s[e]);
          hi = fmax(hi, s[e]);
        }
      lo = wave_min(lo);
      hi = wave_max(hi);
      if (!(lo < hi)) {
        ties = true;
        break;
      }
      // bucket function of this round
      double w = 256.0 / (hi - lo);
      const bool linear = round < 2 && w < 1e300;
      int shift = 0;
      if (!linear) {
        uint64_t kmin = ~0ull, kmax = 0;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if ((member >> e) & 1ull) {
            const uint64_t k = desc_key(s[e]);
            kmin = k < kmin ? k : kmin;
            kmax = k > kmax ? k : kmax;
          }
        kmin = wave_min_u64(kmin);
        kmax = wave_max_u64(kmax);
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
      for (int t = 0; t < 4; ++t) {
        hcnt[lane * 4 + t] = 0u;
        hmass[lane * 4 + t] = 0ull;
      }
      __syncthreads();
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((member >> e) & 1ull) {
          const int b = bucket(s[e]);
          atomicAdd(&hcnt[b], 1u);
          atomicAdd(&hmass[b], (unsigned long long)to_fixed(ev[e]));
        }
      __syncthreads();

      // lane L scans buckets 4L .. 4L+3; inclusive prefix over lanes first
      uint32_t c4[4];
      unsigned long long m4[4];
      uint32_t lc = 0;
      unsigned long long lm = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        c4[t] = hcnt[lane * 4 + t];
        m4[t] = hmass[lane * 4 + t];
        lc += c4[t];
        lm += m4[t];
      }
      uint32_t ic = lc;
      unsigned long long im = lm;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t oc = __shfl_up(ic, o, kWave);
        const unsigned long long om = __shfl_up(im, o, kWave);
        if (lane >= o) {
          ic += oc;
          im += om;
        }
      }
      uint32_t xc = ic - lc;            // exclusive prefix of this lane's first bucket
      unsigned long long xm = im - lm;
      int first = 4;
      uint32_t first_xc = 0;
      unsigned long long first_xm = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bool ok = (cnt_above + (long long)(xc + c4[t]) >= kc) && (mass_above + xm + m4[t] >= target);
        if (ok && first == 4) {
          first = t;
          first_xc = xc;
          first_xm = xm;
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
      }
      const int bstar = 4 * src + __shfl(first, src, kWave);
      cnt_above += (long long)__shfl(first_xc, src, kWave);
      mass_above += __shfl(first_xm, src, kWave);
      const uint32_t n_in = hcnt[bstar];
      __syncthreads();  // everyone has read the histogram before it is cleared
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((member >> e) & 1ull) {
          const int b = bucket(s[e]);
          if (b < bstar) above |= 1ull << e;
          if (b != bstar) member &= ~(1ull << e);
        }
      if (n_in == 1u) {
        take = 1;
        break;
      }
    }
    if (ties) {
      // all members have the same score, hence the same mass u
      unsigned long long u = 0;
      uint32_t nm = 0;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((member >> e) & 1ull) {
          u = to_fixed(ev[e]);
          ++nm;
        }
      u = wave_max_u64(u);
      nm = wave_sum(nm);
      long long need = kc - cnt_above;
      if (mass_above < target && u > 0) {
        const long long need_p = (long long)((target - mass_above + u - 1) / u);
        need = need_p > need ? need_p : need;
      }
      take = need < 0 ? 0 : (need > (long long)nm ? (long long)nm : need);
    }
  }

  // ascending-id compaction: kept = above U (first `take` members by id)
  const uint64_t lt = lanemask_lt();
  long long written = 0, seen = 0;
  int32_t* out = lut + row * (long long)cap;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool is_mem = (member >> e) & 1ull;
    const uint64_t bm = ballot(is_mem);
    const long long rank = seen + __popcll(bm & lt);
    seen += __popcll(bm);
    const bool keep = ((above >> e) & 1ull) || (is_mem && rank < take);
    const uint64_t bk = ballot(keep);
    const long long pos = written + __popcll(bk & lt);
    written += __popcll(bk);
    if (keep && pos < cap) out[pos] = e * kWave + lane;
  }
  if (lane == 0) counts[row] = (int32_t)written;
}

template <int E>
hipError_t launch_e(const double* scores, const Geom& g, int kc, double p, const int32_t* rb,
                    int32_t* lut, int32_t* counts, int cap, hipStream_t s) {
  const long long rows = (long long)g.batch * g.heads * g.nblk;
  select_kernel<E><<<dim3((unsigned)rows), kWave, 0, s>>>(scores, g.nblk, kc, p, rb, lut, counts, cap);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const double* scores, const Geom& g, int kc_default, double p,
                         const int32_t* row_budget, int32_t* lut, int32_t* counts, int cap,
                         hipStream_t s) {
  const int n = g.nblk;
  if (n <= 64) return launch_e<1>(scores, g, kc_default, p, row_budget, lut, counts, cap, s);
  if (n <= 128) return launch_e<2>(scores, g, kc_default, p, row_budget, lut, counts, cap, s);
  if (n <= 256) return launch_e<4>(scores, g, kc_default, p, row_budget, lut, counts, cap, s);
  if (n <= 512) return launch_e<8>(scores, g, kc_default, p, row_budget, lut, counts, cap, s);
  if (n <= 1024) return launch_e<16>(scores, g, kc_default, p, row_budget, lut, counts, cap, s);
  if (n <= 1536) return launch_e<24>(scores, g, kc_default, p, row_budget, lut, counts, cap, s);
  if (n <= 2048) return launch_e<32>(scores, g, kc_default, p, row_budget, lut, counts, cap, s);
  return launch_e<64>(scores, g, kc_default, p, row_budget, lut, counts, cap, s);
}

}  // namespace sa
