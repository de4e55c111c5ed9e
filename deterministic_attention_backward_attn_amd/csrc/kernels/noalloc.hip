// Built-in scratch of dash_attn_bwd_noalloc: the backward's workspace
// (header, order counters, schedule tables, fp32 dQ accumulator) for
// callers that cannot allocate device memory.  One array per GPU, held
// until the process ends; every call on a GPU shares it.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "launch.hpp"

namespace dash {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

// Device address of this GPU's scratch array.  In host code the array's
// name stands for a host-side shadow, so its device address is looked up
// once per device (with that device current) and kept; host code passes
// only that address to kernels and copies.
hipError_t noalloc_scratch(void** out) {
  static std::mutex mu;
  static std::map<int, void*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    it = addr.emplace(dev, p).first;
  }
  *out = it->second;
  return hipSuccess;
}

}  // namespace dash
