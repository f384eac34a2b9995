// copy_probe.hip -- a device-to-device copy kernel used only as a
// measurement anchor: the HBM bandwidth this GPU sustains for a plain
// streaming read + write, against which the library's kernels are compared.
// Built as its own small library (libm3probe.so); not part of libm3ssm's ABI.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;  // 16-byte vectors in flight per thread

// Each workgroup moves kThreads * kVecPerThread consecutive 16-byte vectors;
// every thread issues its loads before its stores.  n16: vectors in total.
__global__ void __launch_bounds__(kThreads) copy_kernel(const v4u* __restrict__ src,
                                                        v4u* __restrict__ dst, size_t n16) {
  const size_t base = (size_t)blockIdx.x * kThreads * kVecPerThread + threadIdx.x;
  v4u v[kVecPerThread];
#pragma unroll
  for (int k = 0; k < kVecPerThread; ++k) {
    const size_t i = base + (size_t)k * kThreads;
    if (i < n16) v[k] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int k = 0; k < kVecPerThread; ++k) {
    const size_t i = base + (size_t)k * kThreads;
    if (i < n16) __builtin_nontemporal_store(v[k], dst + i);
  }
}

}  // namespace

extern "C" {

// Enqueue one copy of `bytes` (a multiple of 16; both pointers 16-byte
// aligned device memory) on `stream`.  Returns 0, or -1 for invalid
// arguments, or the HIP error code of the launch.
int m3probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return -1;
  const size_t n16 = bytes / 16;
  if (n16 == 0) return 0;
  const size_t per = (size_t)kThreads * kVecPerThread;
  const size_t blocks = (n16 + per - 1) / per;
  if (blocks > 0x7fffffffull) return -1;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const v4u*>(src),
                     static_cast<v4u*>(dst), n16);
  return (int)hipGetLastError();
}

}  // extern "C"
