// Static device scratch of the allocation-free key-split entry point
// (fa_fwd_splitkv_noalloc in include/fa_fwd.h).
//
// The array below is the whole scratch: one copy per GPU, created when the
// library's code object is loaded on that GPU and kept until the process
// ends.  Host code never uses the array's name as an address (on the host it
// is only a stand-in for the symbol): the device address is looked up once
// per GPU with hipGetSymbolAddress, with that GPU current, and cached; every
// launch gets the cached pointer.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "fa_internal.h"

namespace fa {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_ptr[kMaxDevices];
std::mutex g_mu;

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
  *ptr = nullptr;
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  // the scratch of the GPU the stream belongs to (the current one for the
  // null stream)
  int dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) {
    *ptr = p;
    return hipSuccess;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  p = g_ptr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace fa
