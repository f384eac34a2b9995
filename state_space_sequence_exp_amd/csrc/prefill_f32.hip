// prefill_f32.hip -- the prefill kernel instantiated for float32 x, B, C,
// every supported rank and head dimension.
#include "prefill_impl.h"

namespace m3 {
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
  return pf::launch_t<float>(a, stream);
}
}  // namespace m3
