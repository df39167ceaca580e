// Device-resident scratch for mamba3_prefill_noalloc: the prefill's segment
// workspace (per-segment summary states, decays and angles of long prompts
// of few chains) in a file-scope device array instead of a caller buffer, for
// callers that cannot allocate device memory.
//
// The array is a device symbol: its host-side name is only a stand-in, so
// host code never passes it to a kernel.  The first call on a device (with
// that device current) resolves the symbol's device address with
// hipGetSymbolAddress and keeps it per device; every later call on that
// device reuses it.  Each GPU holds its own copy of the array for the life of
// the process, and every call on one GPU shares that copy, so calls that
// overlap on one GPU (on different streams, or from different threads)
// race.  No byte of it needs clearing: every value the prefill reads from
// the workspace is written earlier in the same call.
#include <mutex>

#include "m3_kernels.hpp"

namespace m3 {
namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace m3
