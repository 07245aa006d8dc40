// MLA geometry kernels (one 576-wide latent stream shared by all query heads).
#include "vx_internal.h"

namespace vx {

hipError_t launch_scores_mla(const Meta&, const vx_geom&, const void*, const uint16_t*, float,
                             float*, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_attention_mla(const Meta&, const vx_geom&, const void*, const void*,
                                const int32_t*, int, const int32_t*, float, int, int, float*,
                                float*, float*, float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace vx
