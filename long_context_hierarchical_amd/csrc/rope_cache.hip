// RoPE table cache of the decode, prefill and decoding-step calls.
//
// Row p of a RoPE table holds (cos, sin)(p w_i) for the d/2 frequencies w_i = theta^(-2i/d): a
// function of (d, theta) alone, and row p does not depend on how many rows a table has. The array
// below lives in the library's code object (every GPU the library runs on holds its own copy, at
// its own address, until the process ends; nothing is allocated). On each GPU it takes rows
// 0 .. kRopeCacheRows - 1 for the first (d, theta) a call uses there: filled once, on that call's
// stream, and never written again. A later call with the same (d, theta) whose candidate positions
// it covers reads it and launches no table fill; every other call fills the table in its own
// workspace, as before. RECSA_ROPE_CACHE=0 in the environment (read at every call) turns the cache
// off. Host code asks the runtime for the array's device address once per device (with that
// device current) and never passes the array's name to a kernel.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <mutex>

#include "internal.hpp"

namespace recsa {

static __device__ __align__(256) float2 rope_cache[kRopeCacheRows * (kRopeCacheHeadDim / 2)];

namespace {

struct CacheState {
  bool filled = false;   // a fill has been enqueued (its d, theta below)
  bool done = false;     // that fill is known to be complete
  int d = 0;
  uint32_t theta_bits = 0;
  float2* ptr = nullptr;
  hipEvent_t ready = nullptr;
};

constexpr int kMaxDevices = 64;
std::mutex g_mu;
CacheState g_state[kMaxDevices];

}  // namespace

hipError_t rope_cache_table(int d, float theta, const InvFreq& iv, int64_t P, hipStream_t st, const float2** tab) {
  *tab = nullptr;
  if (theta == 0.0f || d > kRopeCacheHeadDim || P < 0 || P >= kRopeCacheRows) return hipSuccess;
  const char* env = std::getenv("RECSA_ROPE_CACHE");
  if (env && env[0] == '0') return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipSuccess;
  uint32_t bits = 0;
  std::memcpy(&bits, &theta, sizeof(bits));
  // a stream under graph capture only reads a cache whose fill has completed; it never fills one
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(st, &cap);
  if (e != hipSuccess) return e;
  const bool capturing = cap != hipStreamCaptureStatusNone;
  std::lock_guard<std::mutex> lock(g_mu);
  CacheState& c = g_state[dev];
  if (!c.filled) {
    if (capturing) return hipSuccess;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(rope_cache));
    if (e != hipSuccess) return e;
    hipEvent_t ev = nullptr;
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    e = launch_rope_table(static_cast<float2*>(p), kRopeCacheRows - 1, d / 2, iv, st);
    if (e == hipSuccess) e = hipEventRecord(ev, st);
    if (e != hipSuccess) {
      (void)hipEventDestroy(ev);
      return e;
    }
    c.filled = true;
    c.d = d;
    c.theta_bits = bits;
    c.ptr = static_cast<float2*>(p);
    c.ready = ev;
    *tab = c.ptr;   // this call runs after the fill on the same stream
    return hipSuccess;
  }
  if (c.d != d || c.theta_bits != bits) return hipSuccess;
  if (!c.done) {
    e = hipEventQuery(c.ready);
    if (e == hipSuccess) {
      c.done = true;
    } else if (e == hipErrorNotReady) {
      // not an error: the runtime may still have recorded it as the thread's last error, which
      // the launch checks after this call read
      (void)hipGetLastError();
      if (capturing) return hipSuccess;
      e = hipStreamWaitEvent(st, c.ready, 0);
      if (e != hipSuccess) return e;
    } else {
      return e;
    }
  }
  *tab = c.ptr;
  return hipSuccess;
}

}  // namespace recsa
