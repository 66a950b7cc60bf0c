// noalloc.hip -- the forward workspace for callers that cannot allocate: a
// file-scope device array of MOE_NOALLOC_SCRATCH_BYTES that every device the
// library runs on holds until the process ends (moe_forward_noalloc).
//
// In host code the array's name is only a host-side stand-in for the symbol:
// its device address comes from hipGetSymbolAddress, once per device with that
// device current, and only that address is ever handed to kernels or copies.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace moe {

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_lock;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null: not looked up)
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_scratch_lock);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
