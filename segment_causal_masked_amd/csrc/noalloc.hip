// Device-resident scratch for callers that cannot allocate (graph capture,
// tight serving loops, harnesses that forbid hipMalloc): the forward's
// workspace (split-piece partials; for sparse plans the selection's sums and
// lists) placed in a fixed file-scope device array instead of caller memory.
//
// The array's name is a host-side stand-in in host code, not a device
// address: its address on a device is taken once per device, with that device
// current, by hipGetSymbolAddress, and only that address is passed to kernels.
// Every call on a device shares its array (it keeps the last call's contents;
// nothing in it needs to start at zero): calls that overlap on one device race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace nomas {
namespace {

__device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

}  // namespace

hipError_t noalloc_scratch(int device, void** ptr) {
  *ptr = nullptr;
  if (device < 0 || device >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;  // resolved with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[device] = p;
  }
  *ptr = g_ptr[device];
  return hipSuccess;
}

}  // namespace nomas
