// Scratch memory of the no-allocation decode entry point
// (starkv_decode_attn_noalloc): a file-scope device array that the library
// owns, so a caller that cannot allocate (code under stream capture, tight
// serving loops, harnesses that forbid allocation) passes only its inputs
// and outputs.  Every GPU the library runs on holds its own copy of the
// array, at its own address, until the process ends.
//
// In host code the array's name stands for a host-side shadow, not for
// device memory: its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// ever handed to kernels.
#include <mutex>

#include "kernels.h"

namespace starkv {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

}  // namespace starkv
