// prefill_bf16_r1_n128.hip -- the prefill kernel instantiated for bfloat16
// x, B, C with MIMO rank 1 and the state size N = 128 fixed at compile time,
// every supported head dimension.  A file of its own: the build schedules it
// with a different instruction-scheduling strategy than the N = 64 kernels.
#include "prefill_impl.h"

namespace m3 {
hipError_t launch_prefill_bf16_r1_n128(const PrefillArgs& a, hipStream_t stream) {
  switch (a.P) {
    case 16: return pf::launch_cfg<pf::Cfg<bf16, 1, 16, 128>>(a, stream);
    case 32: return pf::launch_cfg<pf::Cfg<bf16, 1, 32, 128>>(a, stream);
    case 64: return pf::launch_cfg<pf::Cfg<bf16, 1, 64, 128>>(a, stream);
    case 128: return pf::launch_cfg<pf::Cfg<bf16, 1, 128, 128>>(a, stream);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace m3
