// Library-owned device scratch for the allocation-free GEMM entry point.
//
// One file-scope device array per GPU the library runs on (the HIP runtime
// places it with the code object on each device, so every device holds its
// own copy at its own address until the process ends).  Host code never uses
// the array's name as an address: the device address of the current device's
// copy is looked up once per device with hipGetSymbolAddress and cached.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launchers.h"

namespace bsfp4 {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_device_ptr(void** out) {
  static std::mutex mu;
  static void* ptrs[64] = {nullptr};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

}  // namespace bsfp4
