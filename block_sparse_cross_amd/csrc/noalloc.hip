// Scratch memory of the entry points that allocate nothing (bsx_attn_fwd_noalloc).
//
// The scratch is a file-scope device array: every GPU the library runs on holds its own
// copy, at its own address, from the library's load until the process ends.  In host
// code the array's name is only a stand-in for the symbol, so its device address is
// looked up with hipGetSymbolAddress, once per device, with that device current, and
// kept; kernels and copies get that address, never the name.  Every call on a device
// shares that device's copy: calls that overlap on one GPU race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/bsx.h"
#include "bsx_internal.h"

namespace bsx {
namespace {

static __device__ __align__(256) char scratch[BSX_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

void* noalloc_scratch(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_addr[dev] = ptr;
  }
  *err = hipSuccess;
  return g_addr[dev];
}

}  // namespace bsx
