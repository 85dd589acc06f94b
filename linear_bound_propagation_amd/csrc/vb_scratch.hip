// Fixed device scratch of the allocation-free entry point (vb_crown_noalloc).
//
// The array lives in the library's code object: every GPU the library runs on
// holds its own copy from the time the code object is loaded there until the
// process ends.  Host code never uses the array's name as a device address
// (on the host it is only a stand-in for the symbol); the address is looked up
// once per device with hipGetSymbolAddress, with that device current, and
// cached.
#include <hip/hip_runtime.h>

#include <mutex>

#include "vb_internal.h"

namespace vb {

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};
}  // namespace

hipError_t noalloc_scratch(hipStream_t st, void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace vb
