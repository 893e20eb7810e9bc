// sparse_attn_build_mask without a caller workspace: the float64 block means
// and float32 scores live in a fixed device array of this library, for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops,
// harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ symbol.  On the host its name is only
// a stand-in, so the device address of each GPU's copy is looked up once per
// device with hipGetSymbolAddress (on the first call with that device
// current) and only that address is ever passed to kernels.
//
// The (batch, head) rows are taken in chunks whose means and scores fit the
// array; each chunk runs the pooling, score and selection kernels of
// sparse_attn_build_mask on the caller's stream, so the chunks follow one
// another and reuse the same memory.  Every kernel writes all of the scratch
// it later reads, so nothing has to be cleared between chunks or calls.
// Calls that overlap on one GPU (two streams, or two host threads) share the
// array and race: they must be ordered by the caller.
#include "../../include/sparse_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <mutex>
#include <vector>

#include "sa_launch.h"

int32_t sa_validate_build_mask(const void* qc, const void* kc, const sa_geom* g, int32_t block, double k_frac,
                               double p, const int32_t* row_budget, const int32_t* lut, const int32_t* counts,
                               int32_t cap, sa::Geom& d, int& kcount);
int32_t sa_hip_status(hipError_t e, const char* what);
int32_t sa_fail(int32_t code, const char* msg);

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per GPU
constexpr size_t kAlign = 256;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Device address of this GPU's copy of `scratch`, looked up once per device.
std::mutex g_mu;
std::vector<std::pair<int, void*>> g_addr;

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_mu);
  for (const auto& a : g_addr)
    if (a.first == dev) {
      *out = a.second;
      return hipSuccess;
    }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (ptr == nullptr) return hipErrorInvalidSymbol;
  g_addr.emplace_back(dev, ptr);
  *out = ptr;
  return hipSuccess;
}

// Scratch bytes of `heads` (batch, head) rows: block means of Q and K
// [heads, nblk, d], float64, and the scores [heads, nblk, nblk], float32,
// each region 256-byte aligned.
size_t chunk_bytes(const sa::Geom& d, size_t heads) {
  const size_t n = (size_t)d.nblk;
  return 2 * round_up(heads * n * d.d * sizeof(double)) + round_up(heads * n * n * sizeof(float));
}

}  // namespace

extern "C" size_t sparse_attn_build_mask_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int32_t sparse_attn_build_mask_noalloc(const void* qc, const void* kc, const sa_geom* g,
                                                  int32_t block, double k_frac, double p,
                                                  const int32_t* row_budget, int32_t* lut, int32_t* counts,
                                                  int32_t cap, void* stream) {
  sa::Geom d;
  int kcount = 0;
  const int32_t v = sa_validate_build_mask(qc, kc, g, block, k_frac, p, row_budget, lut, counts, cap, d, kcount);
  if (v != SA_OK) return v;
  const size_t per_head = chunk_bytes(d, 1);
  if (per_head > kScratchBytes) {
    char msg[200];
    std::snprintf(msg, sizeof(msg),
                  "one (batch, head) needs %zu bytes of scratch (%d blocks, head_dim %d), above the %zu of "
                  "the allocation-free form",
                  per_head, d.nblk, d.d, kScratchBytes);
    return sa_fail(SA_ERR_CAPACITY, msg);
  }
  void* base = nullptr;
  hipError_t e = scratch_address(&base);
  if (e != hipSuccess) return sa_hip_status(e, "scratch symbol address");
  const int rows = d.batch * d.heads;
  int chunk = (int)(kScratchBytes / per_head) < rows ? (int)(kScratchBytes / per_head) : rows;
  while (chunk > 1 && chunk_bytes(d, (size_t)chunk) > kScratchBytes) --chunk;
  const size_t n = (size_t)d.nblk;
  const size_t head_c = (size_t)d.n_pad * d.d * 2;   // bytes of one cube-major head
  const double scale = 1.0 / std::sqrt((double)d.d);
  hipStream_t s = (hipStream_t)stream;
  for (int r0 = 0; r0 < rows; r0 += chunk) {
    const int nr = rows - r0 < chunk ? rows - r0 : chunk;
    sa::Geom gc = d;
    gc.batch = 1;
    gc.heads = nr;
    char* ws = static_cast<char*>(base);
    double* qbar = reinterpret_cast<double*>(ws);
    double* kbar = reinterpret_cast<double*>(ws + round_up((size_t)nr * n * d.d * sizeof(double)));
    float* sc = reinterpret_cast<float*>(ws + 2 * round_up((size_t)nr * n * d.d * sizeof(double)));
    const char* q = static_cast<const char*>(qc) + (size_t)r0 * head_c;
    const char* k = static_cast<const char*>(kc) + (size_t)r0 * head_c;
    e = sa::launch_pool(q, k, qbar, kbar, gc, s);
    if (e != hipSuccess) return sa_hip_status(e, "pool launch");
    e = sa::launch_block_scores(qbar, kbar, sc, scale, gc, s);
    if (e != hipSuccess) return sa_hip_status(e, "block score launch");
    e = sa::launch_select(sc, gc, kcount, p, row_budget ? row_budget + (size_t)r0 * n : nullptr,
                          lut + (size_t)r0 * n * cap, counts + (size_t)r0 * n, cap, s);
    if (e != hipSuccess) return sa_hip_status(e, "select launch");
  }
  return sa_hip_status(hipSuccess, "");
}
