// noalloc_scratch.hip -- the library's static device scratch array, used by qv_w4a4_linear_noalloc
// (callers that cannot allocate device memory).  The array holds the packed activation codes and
// the per-row scales that qv_w4a4_linear keeps in the caller's workspace.
//
// Each GPU the library runs on holds its own copy of the array (its size is QV_NOALLOC_SCRATCH_BYTES)
// from the moment the library's code object is loaded on that device until the process ends.  In
// host code the array's name is only a host-side stand-in: the device address of a GPU's copy is
// looked up here with hipGetSymbolAddress, once per device with that device current, and every
// kernel argument uses that address.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "qv.h"
#include "qv_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[QV_NOALLOC_SCRATCH_BYTES];

// Device addresses of the array, per device ordinal below kCachedDevices (higher ordinals look the
// address up on every call).  Concurrent first calls from several host threads store the same value.
constexpr int kCachedDevices = 64;
std::atomic<void*> g_scratch[kCachedDevices];

}  // namespace

namespace qv {

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cacheable = dev >= 0 && dev < kCachedDevices;
  void* p = cacheable ? g_scratch[dev].load(std::memory_order_acquire) : nullptr;
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    if (cacheable) g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  *bytes = QV_NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace qv
