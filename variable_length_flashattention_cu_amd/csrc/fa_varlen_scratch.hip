// fa_varlen_scratch.hip -- the static device scratch of fa_varlen_fwd_noalloc:
// the work-item map of one forward call, held in a file-scope device array so
// that the call allocates nothing.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address on the current GPU comes from hipGetSymbolAddress, taken once
// per device (every GPU holds its own copy of the array) and cached here.
// Only that address is ever handed to kernels.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "fa_varlen_launch.h"

static __device__ __align__(256) int32_t scratch[fa::kNoAllocMaxBatch + 1];

namespace fa {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<int32_t*> g_scratch[kMaxDevices];

}  // namespace

hipError_t noalloc_map_scratch(int32_t** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int32_t* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // first call on this device (the device is current): its copy's address
    e = hipGetSymbolAddress(reinterpret_cast<void**>(&p), HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace fa
