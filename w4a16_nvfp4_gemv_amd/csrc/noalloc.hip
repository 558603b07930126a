// Library-owned scratch of the entry point that allocates nothing
// (nvfp4_gemv_splitk_noalloc): the FP32 partial sums and arrival counters of
// the cross-workgroup split-K GEMV live in a file-scope device array instead
// of a caller workspace.  Each GPU holds its own copy of the array, created
// when the library's code object is loaded on that device and kept until
// the process ends; its address on a device is looked up once, with that
// device current, and only that address is passed to kernels (the array's
// name is a host-side stand-in in host code).
//
// The array starts zero-filled, and every split-K call leaves its counter
// words zero again, so no clearing is needed between calls.  All calls on
// one GPU share the array: calls that overlap (on different streams) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace w4a16 {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace w4a16
