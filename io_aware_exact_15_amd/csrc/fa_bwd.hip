// Backward pass (placeholder until the kernels land).
#include "fa_device.hpp"
#include "fa_internal.h"
#include "../../include/fa.h"

namespace fa {
int launch_backward(const void*, const void*, const void*, const void*, int, const void*, const float*, float*,
                    float*, float*, float*, int, int, int, int, float, int, hipStream_t) {
  return FA_ERR_UNSUPPORTED;
}
}  // namespace fa
