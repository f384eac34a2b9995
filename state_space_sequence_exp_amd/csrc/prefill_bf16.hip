// prefill_bf16.hip -- the prefill kernel instantiated for bfloat16 x, B, C
// (fp32 state and accumulation), every supported rank and head dimension.
#include "prefill_impl.h"

namespace m3 {
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  return pf::launch_t<bf16>(a, stream);
}
}  // namespace m3
