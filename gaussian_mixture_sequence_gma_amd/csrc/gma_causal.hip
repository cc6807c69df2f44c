// Causal GMA forward (chunked prefix scan) -- not yet implemented.
#include "gma_device.h"
#include "gma_internal.h"

namespace gma {
hipError_t launch_causal(const Plan&, const Tensors&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace gma
