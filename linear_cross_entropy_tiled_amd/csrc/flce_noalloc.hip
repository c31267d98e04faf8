// flce_forward_no_alloc: the forward pass for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The forward pass's scratch -- the status word, the
// per-split softmax partials and the per-block sums that flce_forward keeps in
// its workspace -- lives instead in a fixed file-scope device array, one copy
// per GPU, which the library looks up once per device and never frees.  The
// kernels are flce_forward's; every call on a GPU shares that GPU's array, so
// calls that overlap on one GPU race.  Nothing in the array has to start at
// zero: every launch writes each partial it later reads.
#include <mutex>

#include "flce_internal.h"

namespace flce {
// 8 MiB: the forward scratch is 20 bytes per padded row per vocabulary split
// (about 256 row tiles x splits in total) plus 24 bytes per 256 rows, so this
// covers N up to ~400k tokens at any vocabulary size.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
}  // namespace flce

static __device__ __align__(256) char scratch[flce::kNoAllocScratchBytes];

namespace flce {
namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

// Device address of the current GPU's copy of `scratch`, looked up on the first
// call on that GPU (with it current).  Host code never passes the array's name
// itself: on the host that is only a stand-in for the symbol.
static hipError_t current_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev],
                 [dev] { g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch)); });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace flce

using namespace flce;

extern "C" int flce_forward_no_alloc(const flce_params* p, const void* hidden, const void* weight, const void* bias,
                                     const void* targets, float* loss, float* lse, int64_t* num_correct,
                                     float* entropy_sum, void* stream) {
  Plan pl;
  const int rc = make_plan(p, &pl);
  if (rc != FLCE_OK) return rc;
  pl.has_bias = bias != nullptr;
  if (!loss && (pl.reduction != FLCE_REDUCTION_NONE || pl.N > 0)) return FLCE_ERR_INVALID_ARG;
  if (pl.N > 0 && (!hidden || !targets || !lse)) return FLCE_ERR_INVALID_ARG;
  if (!weight) return FLCE_ERR_INVALID_ARG;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(hidden) | reinterpret_cast<uintptr_t>(weight) |
                        reinterpret_cast<uintptr_t>(bias) | reinterpret_cast<uintptr_t>(targets);
  if ((mis & 15) != 0) return FLCE_ERR_UNSUPPORTED;
  if (pl.f_bytes > kNoAllocScratchBytes) return FLCE_ERR_UNSUPPORTED;   // beyond the fixed scratch
  // the stream must belong to the current GPU, whose copy of the scratch is used
  int cur = 0;
  hipDevice_t sdev = 0;
  if (hipGetDevice(&cur) != hipSuccess) return FLCE_ERR_HIP;
  if (stream && hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return FLCE_ERR_HIP;
  if (stream && sdev != cur) return FLCE_ERR_INVALID_ARG;
  void* ws = nullptr;
  if (current_scratch(&ws) != hipSuccess) return FLCE_ERR_HIP;
  const hipError_t e = launch_forward(pl, hidden, weight, bias, targets, loss, lse, num_correct, entropy_sum,
                                      static_cast<char*>(ws), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}
