// scratch.hip -- device-resident scratch of the no-allocation sparse-layer entry point
// (hs_sparse_attn_gather_noalloc): the split partials that the other entry points keep in the
// caller's workspace live here instead, so that a caller that cannot allocate device memory
// (code under graph capture, tight serving loops) can still run the layer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "hs_kernels.h"

namespace hs {

// One copy per device, loaded with the library's code and held until the process ends.  In host
// code `scratch` names a host-side stand-in: kernels get the address from scratch_buffer.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_buffer(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {  // first call on this device (it is the current device here)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace hs
