// Backward pass (placeholder until the kernels land).
#include <hip/hip_runtime.h>

#include "bsx_internal.h"

namespace bsx {

hipError_t launch_bwd_bf16(const BwdParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace bsx
