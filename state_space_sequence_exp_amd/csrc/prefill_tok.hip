// prefill_tok.hip -- the token-lane prefill kernel (prefill_tok.h)
// instantiated for the shape it takes: bfloat16 x, B, C, rank 1, 64-token
// chunks, state size 64 and head dimension 64.
#include "prefill_tok.h"

namespace m3 {
hipError_t launch_prefill_tok(const PrefillArgs& a, hipStream_t stream, bool* taken) {
  return pt::tok_dispatch(a, stream, taken);
}
}  // namespace m3
