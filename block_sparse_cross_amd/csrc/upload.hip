// Moves a small host-built descriptor into the caller's workspace through kernel
// arguments.  The arguments are captured when the kernel is enqueued, so the copy
// is ordered on the caller's stream, never waits for the host, and the host buffer
// is free as soon as the call returns.
#include <hip/hip_runtime.h>

#include "bsx_internal.h"

namespace bsx {
namespace {

struct UploadPayload {
  uint32_t words[kUploadWords];
};

__global__ __launch_bounds__(256) void upload_kernel(UploadPayload payload, uint32_t* dst, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = payload.words[i];
}

}  // namespace

hipError_t launch_upload(const uint32_t* host_words, size_t n_words, uint32_t* dst,
                         hipStream_t stream) {
  for (size_t base = 0; base < n_words; base += kUploadWords) {
    const int n = int(n_words - base < size_t(kUploadWords) ? n_words - base : kUploadWords);
    UploadPayload payload;
    for (int i = 0; i < n; ++i) payload.words[i] = host_words[base + i];
    hipLaunchKernelGGL(upload_kernel, dim3(1), dim3(256), 0, stream, payload, dst + base, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bsx
