// Split-K decode attention on the int4 cache, matrix-core variant (pending).
#include "kvq_internal.h"

namespace kvq {

bool mfma_supports(int, int, int, int) { return false; }

hipError_t launch_partial_mfma(const PartialArgs &, int, int, int, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace kvq
