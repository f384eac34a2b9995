// copy_probe.hip -- device-to-device copy kernels used only as a measurement
// anchor: the HBM bandwidth this GPU sustains for a plain streaming read +
// write, against which the library's kernels are compared.  A few plain
// variants (vectors in flight per thread, ordinary or non-temporal accesses)
// are compiled, since which of them runs fastest is a property of the chip
// and is measured, not assumed; the anchor is the best of them.  Built as
// its own small library (libm3probe.so); not part of libm3ssm's ABI.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

// Each workgroup moves kThreads * V consecutive 16-byte vectors; every thread
// issues its V loads before its stores.  n16: vectors in total.
template <int V, bool kNT>
__global__ void __launch_bounds__(kThreads) copy_kernel(const v4u* __restrict__ src,
                                                        v4u* __restrict__ dst, size_t n16) {
  const size_t base = (size_t)blockIdx.x * kThreads * V + threadIdx.x;
  v4u v[V];
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const size_t i = base + (size_t)k * kThreads;
    if (i < n16) v[k] = kNT ? __builtin_nontemporal_load(src + i) : src[i];
  }
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const size_t i = base + (size_t)k * kThreads;
    if (i < n16) {
      if (kNT)
        __builtin_nontemporal_store(v[k], dst + i);
      else
        dst[i] = v[k];
    }
  }
}

template <int V, bool kNT>
int launch(const void* src, void* dst, size_t n16, hipStream_t stream) {
  const size_t per = (size_t)kThreads * V;
  const size_t blocks = (n16 + per - 1) / per;
  if (blocks > 0x7fffffffull) return -1;
  hipLaunchKernelGGL((copy_kernel<V, kNT>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const v4u*>(src), static_cast<v4u*>(dst), n16);
  return (int)hipGetLastError();
}

}  // namespace

extern "C" {

// Number of copy variants m3probe_copy takes.
int m3probe_copy_variants(void) { return 6; }

// Enqueue one copy of `bytes` (a multiple of 16; both pointers 16-byte
// aligned device memory) on `stream` with copy variant `variant` (0 ..
// m3probe_copy_variants() - 1: 4, 8 or 16 vectors per thread, each with
// ordinary then non-temporal accesses).  Returns 0, or -1 for invalid
// arguments, or the HIP error code of the launch.
int m3probe_copy(const void* src, void* dst, size_t bytes, int variant, void* stream) {
  if (!src || !dst || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return -1;
  const size_t n16 = bytes / 16;
  if (n16 == 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (variant) {
    case 0: return launch<4, false>(src, dst, n16, s);
    case 1: return launch<4, true>(src, dst, n16, s);
    case 2: return launch<8, false>(src, dst, n16, s);
    case 3: return launch<8, true>(src, dst, n16, s);
    case 4: return launch<16, false>(src, dst, n16, s);
    case 5: return launch<16, true>(src, dst, n16, s);
    default: return -1;
  }
}

}  // extern "C"
