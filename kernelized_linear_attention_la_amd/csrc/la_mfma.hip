// bf16 matrix-core (MFMA) chunkwise kernels for gfx950.
#include "la_device.h"
#include "la_internal.h"

namespace la {

bool mfma_supported(const Shape &, int) { return false; }

hipError_t launch_mfma(const FwdArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace la
