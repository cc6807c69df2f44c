// Projection GEMM for the GMA layer -- not yet implemented.
#include "gma_device.h"
#include "gma_internal.h"

namespace gma {
hipError_t launch_proj(const void*, const void*, int64_t, int, int, int, int, int64_t, float*,
                       hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace gma
