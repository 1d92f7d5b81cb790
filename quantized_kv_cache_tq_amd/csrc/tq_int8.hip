// tq_int8.hip -- placeholder until the int8 prompt-attention kernel lands.
#include "tq_common.h"
#include "tq_launch.h"

namespace tq {

hipError_t plan_int8(int64_t, int32_t, int32_t, int64_t, Int8Plan *p) {
  *p = Int8Plan{};
  return hipErrorNotSupported;
}

hipError_t launch_int8(const float *, int64_t, int32_t, const int8_t *, const int8_t *,
                       const uint16_t *, const uint16_t *, int32_t, const int32_t *, int64_t,
                       int64_t, int64_t, float, float *, void *, const Int8Plan &, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace tq
