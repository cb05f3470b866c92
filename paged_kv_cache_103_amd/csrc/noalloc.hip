// Device scratch of pa_decode_noalloc (include/pa.h): the split-K summaries
// of a decode call for callers that cannot allocate device memory. The array
// is part of the library's code object, so each GPU the library runs on
// holds its own copy, at its own address, until the process ends.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "pa_internal.h"

namespace pa {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

// This GPU's address of the array (the host-side name `scratch` is only a
// stand-in: a kernel handed it would fault). Looked up once per device, with
// that device current.
void* noalloc_scratch(hipError_t* err) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> ptrs[kMaxDevices];
  static std::mutex init;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(init);
    p = ptrs[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) {
        *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
        return nullptr;
      }
      ptrs[dev].store(p, std::memory_order_release);
    }
  }
  *err = hipSuccess;
  return p;
}

}  // namespace pa
