// prefill.hip -- host side of the chunked prefill (segment sizing, dispatch to the per-type
// kernels of prefill_bf16_r*.hip and prefill_f32.hip, whose body is prefill_impl.h) and two
// small kernels: the empty-sequence final state and the continuation entry state.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

// h_final of an empty sequence: the given initial state, or zero.  dst may
// equal src.
__global__ void copy_or_zero_kernel(float* dst, const float* src, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src ? src[i] : 0.f;
}

// Entry state of each sequence's first chunk when the sequence continues
// from a given state h0 and previous token (x_prev, B_prev):
// G = h0 + (1 - lam_0) dt_0 B_prev x_prev^T, the state plus the trapezoid's
// previous-input term, which the first token's update decays and rotates
// together.  Written to the workspace's entry states, where the prefill
// kernel's first segment (and the look-back of later ones) reads it.  One
// thread per state element.
template <typename T>
__global__ void entry_kernel(PrefillArgs a) {
  const size_t np = (size_t)a.N * a.P;
  const size_t total = (size_t)a.nb * a.H * np;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t bh = i / np, e = i % np;
    const int n = (int)(e / a.P), p = (int)(e % a.P);
    float v = a.h0 ? a.h0[i] : 0.f;
    if (a.x_prev) {
      const int b = (int)(bh / a.H), h = (int)(bh % a.H);
      const size_t tok0 = (size_t)b * a.T * a.H + h;  // the sequence's first token
      const float w0 = a.lam ? (1.f - a.lam[tok0]) * a.dt[tok0] : 0.f;
      const T* xp = static_cast<const T*>(a.x_prev) + bh * a.R * a.P;
      const T* bp = static_cast<const T*>(a.B_prev) + bh * a.R * a.N;
      float acc = 0.f;
      for (int r = 0; r < a.R; ++r)
        acc = __builtin_fmaf(to_f32(bp[r * a.N + n]), to_f32(xp[r * a.P + p]), acc);
      v = __builtin_fmaf(w0, acc, v);
    }
    a.cont_entry[bh * np + prefill_state_index(a.N, n, p)] = v;
  }
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
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                       dim3(256), 0, stream, a.h_final, a.h0, n);
    return hipGetLastError();
  }
  if (a.h0 || a.x_prev) {
    const size_t n = (size_t)a.nb * a.H * a.N * a.P;
    const size_t blocks = (n + 255) / 256;
    const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
    if (dtype == M3_BF16)
      hipLaunchKernelGGL(entry_kernel<bf16>, grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(entry_kernel<float>, grid, dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dtype != M3_BF16) return launch_prefill_f32(a, stream);
  // the token-lane kernel where it takes the shape (bfloat16, rank 1, 64-token
  // chunks, N = P = 64; its y stores are 8-byte vectors)
  if (reinterpret_cast<uintptr_t>(a.y) % 8 == 0) {
    bool taken = false;
    const hipError_t e = launch_prefill_tok(a, stream, &taken);
    if (taken) return e;
  }
  switch (a.R) {
    case 1: return launch_prefill_bf16_r1(a, stream);
    case 2: return launch_prefill_bf16_r2(a, stream);
    case 4: return launch_prefill_bf16_r4(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace m3
