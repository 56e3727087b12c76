// Fixed device scratch for the allocation-free backward entry point.
//
// The backward's workspace (one fp32 dgamma partial row per partition block,
// then a 16-byte record per row for rows that may take the two-pass tier)
// lives here, in a file-scope device array that every GPU the library runs on
// holds from the module's load to the end of the process. Host code never
// uses the array's name as an address: its per-device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is passed to the kernels.
//
// Every call on one GPU shares that GPU's copy, which keeps whatever the last
// call left in it. The backward reads nothing from its workspace that the
// same call did not write first, so nothing is cleared; two calls that
// overlap in time on one GPU race on the array.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "launch.hpp"
#include "rmsnorm_mi355x.h"

namespace {

static_assert(RMSN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[RMSN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

}  // namespace

namespace rmsn {

hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace rmsn
