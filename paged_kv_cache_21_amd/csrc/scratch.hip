// Fixed device scratch for the decode entry point that allocates nothing
// (pkv_paged_decode_attn_noalloc): the split-K partial results live in a
// file-scope device array instead of a caller workspace.  Each device the
// library runs on holds its own copy of the array, at its own address, until the
// process ends.  The array's name is a host-side stand-in in host code; its device
// address is taken once per device with hipGetSymbolAddress (that device current)
// and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace pkv {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace pkv
