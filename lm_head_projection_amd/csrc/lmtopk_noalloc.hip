// lmtopk_noalloc.hip - the scratch memory of lmtopk_binary_noalloc, the binary
// entry point for callers that cannot allocate device memory (code under
// graph capture, tight serving loops): its workspace is one file-scope device
// array per GPU instead of a caller's buffer.
#include <hip/hip_runtime.h>
#include <mutex>
#include <stdint.h>

#include "lmtopk.h"
#include "lmtopk_internal.hpp"

namespace lmtopk {

// Every GPU the library runs on holds one copy until the process ends.  Calls
// on one GPU share it and overlapping calls on one GPU race; each call leaves
// its completion counter and key histograms (the first kCounterBytes +
// kHistBytes bytes) at zero, which the first use on a device sets up.
static __device__ __align__(256) uint8_t scratch[LMTOPK_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // device address of `scratch` on each device
}  // namespace

int noalloc_scratch(void** ptr, void* stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    // `scratch` in host code is only a stand-in for the symbol; its device
    // address, per device, comes from the runtime (with that device current)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    const int z = launch_zero(p, kCounterBytes + kHistBytes, stream);
    if (z != 0) return z;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return 0;
}

}  // namespace lmtopk
