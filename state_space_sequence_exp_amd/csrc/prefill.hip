// prefill.hip -- host side of the chunked prefill: segment sizing and dispatch to the per-type kernels (prefill_bf16_r*.hip,
// prefill_f32.hip; the kernel itself is in prefill_impl.h).
#include "m3_internal.h"

namespace m3 {
namespace {

__global__ void fill_zero_kernel(float* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace

// Chunks per segment: enough segments for about one workgroup per CU (256 on
// MI355X) across all sequences; longer segments amortise each segment's
// extra local pass and chain step.
int prefill_segment_chunks(int nb, int H, int nC) {
  const long units = (long)nb * H;
  const long target = 256;
  long k = (nC * units + target - 1) / target;
  if (k < 1) k = 1;
  if (k > nC) k = nC;
  return (int)k;
}

hipError_t launch_prefill(const PrefillArgs& a, m3_dtype dtype, hipStream_t stream) {
  if (a.nb == 0) return hipSuccess;
  if (a.T == 0) {
    if (!a.h_final) return hipSuccess;
    const size_t n = (size_t)a.nb * a.H * a.N * a.P;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       a.h_final, n);
    return hipGetLastError();
  }
  if (dtype != M3_BF16) return launch_prefill_f32(a, stream);
  switch (a.R) {
    case 1: return launch_prefill_bf16_r1(a, stream);
    case 2: return launch_prefill_bf16_r2(a, stream);
    case 4: return launch_prefill_bf16_r4(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace m3
