// prefill_bf16_r1.hip -- the prefill kernel instantiated for bfloat16 x, B, C
// (fp32 state and accumulation) with MIMO rank 1, every supported head
// dimension.
#include "prefill_impl.h"

namespace m3 {
hipError_t launch_prefill_bf16_r1(const PrefillArgs& a, hipStream_t stream) {
  return pf::launch_tr<bf16, 1>(a, stream);
}
}  // namespace m3
