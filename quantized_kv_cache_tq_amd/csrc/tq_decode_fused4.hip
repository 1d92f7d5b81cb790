// tq_decode_fused4.hip -- the fused decode kernel's one-block variants
// (64-key blocks per wave, no next-block prefetch: single-row decodes whose
// splits fit one round of workgroups, the 32K shapes among them), compiled
// in a translation unit of their own so that they can take the compiler's
// instruction-level-parallelism scheduling strategy.  Measured in one
// process (24-layer graphs, 32 q / 4 kv heads, 32K cells): 316.8 -> 309.8 us;
// the same strategy made the prefetching variants slower, so only these take
// it.  The kernel itself is the one in tq_decode.hip.
#define TQ_DECODE_FUSED_BLOCK4_TU
#include "tq_decode.hip"

namespace tq {

#define TQ_FUSED_PARAMS                                                                                     \
  const uint8_t *, const uint16_t *, const uint8_t *, const uint16_t *, int64_t, const int64_t *,        \
      const int32_t *, int64_t, const void *, int, int, int, int, int, float, float, float *, int
template __global__ void decode_fused_kernel<2, 4, true, false>(TQ_FUSED_PARAMS);
template __global__ void decode_fused_kernel<2, 4, false, false>(TQ_FUSED_PARAMS);
template __global__ void decode_fused_kernel<3, 4, true, false>(TQ_FUSED_PARAMS);
template __global__ void decode_fused_kernel<3, 4, false, false>(TQ_FUSED_PARAMS);
template __global__ void decode_fused_kernel<4, 4, true, false>(TQ_FUSED_PARAMS);
template __global__ void decode_fused_kernel<4, 4, false, false>(TQ_FUSED_PARAMS);
#undef TQ_FUSED_PARAMS

}  // namespace tq
