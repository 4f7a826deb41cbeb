// Device scratch of the allocation-free decode entry point (recsa_decode_noalloc).
//
// The array below lives in the library's code object: every GPU the library runs on holds its
// own copy, at its own address, until the process ends. Host code never passes the array's
// name to a kernel (on the host that name is only a stand-in); it asks the runtime for the
// device address once per device, with that device current, and uses that address for every
// launch. Calls that use the scratch on one GPU share it: calls that overlap in time on one GPU
// race on its contents.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.hpp"

namespace recsa {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

hipError_t noalloc_scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace recsa
