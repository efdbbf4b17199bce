// Fixed device scratch for scan_topk_noalloc: the workspace of a top-k step
// held in a file-scope device array, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// Each GPU the library runs on holds its own copy of `scratch` from the moment
// the code object is loaded until the process ends.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.
#include <mutex>

#include "fathom_internal.h"

namespace fathom {
namespace {

__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // per device: the device address of `scratch` (null before the first call)

}  // namespace

hipError_t noalloc_scratch(void** out) {
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
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace fathom
