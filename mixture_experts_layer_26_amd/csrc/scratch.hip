// The fixed scratch buffer of moe_grouped_ffn_noalloc: device memory that is part of the
// code object, so a call needs no allocation (for callers that cannot allocate: code
// under HIP graph capture, serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope __device__ array. In host code its name is only a host-side
// stand-in for the symbol, not a device address, so host code never passes it to a kernel
// or a copy: the address is taken once per device with hipGetSymbolAddress, with that
// device current, and kept. Each device holds its own copy of the array (at its own
// address) until the process ends, and every call on a device shares that device's copy.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace moe {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {nullptr};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
