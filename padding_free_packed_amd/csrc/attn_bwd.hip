// Backward of packed attention (being written; returns hipErrorNotSupported).
#include "common.h"
#include "kernels.h"

namespace pe {

hipError_t launch_attn_bwd(bool, int, const void*, const void*, const void*, const void*, const void*,
                           const float*, const int32_t*, const int32_t*, int32_t, int32_t, int32_t, float,
                           void*, void*, void*, float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace pe
