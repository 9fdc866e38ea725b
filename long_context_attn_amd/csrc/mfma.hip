// bf16 MFMA kernels of the Lightning Attention layer (placeholder until written).
#include "la_internal.h"

namespace la {
bool mfma_supported(const PrefillArgs&) { return false; }
hipError_t launch_chunk_state_mfma(const PrefillArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_walk_mfma(const PrefillArgs&, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace la
