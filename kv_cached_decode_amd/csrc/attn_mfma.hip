// attn_mfma.hip -- placeholder until the matrix-core verify kernel lands.
#include "kvd_internal.h"

namespace kvd {

bool mfma_supported(int, int, int) { return false; }
int mfma_step_keys() { return 256; }
hipError_t launch_attn_mfma(const AttnArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace kvd
