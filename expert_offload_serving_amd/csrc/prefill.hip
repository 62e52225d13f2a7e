// Prefill forward (grouped MFMA GEMMs, double-buffered layer uploads).
#include "moe_internal.h"

namespace moe {

hipError_t prefill_forward(Ctx*, int, const void* const*, int, const float* const*, void* const*,
                           float* const*, hipStream_t) {
  return hipErrorNotSupported;
}

void prefill_free(Ctx*) {}

}  // namespace moe
