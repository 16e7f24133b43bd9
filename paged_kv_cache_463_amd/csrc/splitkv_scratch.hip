// Static device scratch of the allocation-free split-KV entry point
// (pa_decode_splitkv_noalloc): the partial rows, (max, normaliser) pairs and
// work counter that pa_decode_splitkv carves out of a caller's workspace live
// here instead, in a file-scope device array that every GPU the library runs
// on holds until the process ends.
//
// In host code the array's name is only a host-side stand-in: its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and only that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "pa_launch.h"

namespace pa {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t scratch_device_ptr(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace pa
