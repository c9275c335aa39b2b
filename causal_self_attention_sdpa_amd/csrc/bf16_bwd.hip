#include "gattn_internal.h"
namespace gattn {
hipError_t bf16_bwd_main(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                         const float*, const float*, float*, uint16_t*, uint16_t*, int, int, int,
                         float, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace gattn
