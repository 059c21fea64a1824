// Library-owned scratch for the allocation-free W8A8_INT8 layer
// (mq_w8a8_linear_noalloc): the per-token quantizer's codes and scales for
// more than one token live in a fixed device array instead of a caller's
// workspace. Each GPU the library runs on holds its own copy of the array
// (the code object is loaded per device) until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress and
// only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

static __device__ __align__(256) uint8_t scratch[mq::kNoallocScratchBytes];

namespace mq {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current: this device's copy
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace mq
