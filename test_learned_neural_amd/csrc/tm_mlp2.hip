// Specialised MFMA kernel for the 2-layer d=64 hidden=256 memory (placeholder
// until the kernel lands: reports the shape as unsupported).
#include "tm_internal.h"

namespace titans {

bool mlp2_supported(const Shape&, int) { return false; }
int64_t mlp2_ws_bytes(const Shape&, int) { return 0; }
hipError_t launch_mlp2(const Shape&, int, const void*, const void*, const void*, const float*,
                       const float*, const float*, const float*, const float*, void*, float*,
                       float*, void*, hipStream_t) {
  return hipErrorInvalidConfiguration;
}

}  // namespace titans
