// block.hip -- the block-side steps on either side of the SSM (Mamba-3 paper
// translation, section 3.4; the reading of the projections is stated in
// include/m3ssm.h):
//
//   pre-pass   B~ = RMSNorm_N(B) * wB[h] + bB[h,r],  C~ likewise   (BCNorm + bias)
//              X[r] = x * U[h,r]                                   (MIMO up-projection)
//   post-pass  y_out = sum_r D[h,r] * y[r]                         (MIMO down-projection)
//
// Both passes stream their operands once and are bound by HBM bandwidth, so
// they are laid out for coalescing rather than for the matrix cores: lanes
// move 16-byte vectors (8 bfloat16 or 4 float), consecutive lanes
// consecutive vectors, each thread kU of them a grid-stride apart with all
// loads issued first.  The pre-pass is one launch over three row spaces
// (blockIdx.y: B rows, C rows, x rows); a B or C row of N channels is N / E
// consecutive lanes (E elements per vector, N / E a power of two dividing the
// wave), whose sum of squares is reduced by lane shuffles inside that group.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

constexpr int kBlkThreads = 256;

template <typename T>
struct Vec16 {
  static constexpr int E = 16 / sizeof(T);
};

__device__ __forceinline__ void unpack16(const uint4 w, float (&v)[8], const bf16*) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(ws[i] << 16);
    v[2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(const uint4 w, float (&v)[4], const float*) {
  v[0] = __uint_as_float(w.x);
  v[1] = __uint_as_float(w.y);
  v[2] = __uint_as_float(w.z);
  v[3] = __uint_as_float(w.w);
}
__device__ __forceinline__ uint4 pack16(const float (&v)[8], const bf16*) {
  uint32_t ws[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 p = {from_f32<bf16>(v[2 * i]), from_f32<bf16>(v[2 * i + 1])};
    ws[i] = __builtin_bit_cast(uint32_t, p);
  }
  return make_uint4(ws[0], ws[1], ws[2], ws[3]);
}
__device__ __forceinline__ uint4 pack16(const float (&v)[4], const float*) {
  return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                    __float_as_uint(v[3]));
}

// Vectors per thread: each thread handles kU vectors a grid-stride apart
// (the stride is a multiple of the wave, so a row's lane group stays in one
// wave), issuing all their loads before any arithmetic.
constexpr int kU = 4;

template <typename T>
__global__ void __launch_bounds__(kBlkThreads) prepass_kernel(BlockArgs a) {
  constexpr int E = Vec16<T>::E;
  const size_t stride = (size_t)gridDim.x * kBlkThreads;
  const size_t i0 = (size_t)blockIdx.x * kBlkThreads + threadIdx.x;  // first vector
  const int part = blockIdx.y;
  if (part < 2) {
    // BCNorm + bias on 16-byte pieces of B or C rows
    const int cpr = a.N / E;  // lanes per row: a power of two that divides the wave
    const size_t nvec = a.rows * a.R * (size_t)cpr;
    const uint4* src = static_cast<const uint4*>(part == 0 ? a.B : a.C);
    uint4* dst = static_cast<uint4*>(part == 0 ? a.B_out : a.C_out);
    const float* wbase = part == 0 ? a.norm_B : a.norm_C;
    const float* bbase = part == 0 ? a.bias_B : a.bias_C;
    uint4 raw[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t i = i0 + u * stride;
      raw[u] = i < nvec ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
    float w[kU][E], b[kU][E];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t i = i0 + u * stride;
      const size_t row = i < nvec ? i / cpr : 0;  // (token, head, rank) row
      const int n0 = (int)(i % cpr) * E;
      const int r = (int)(row % a.R), h = (int)((row / a.R) % a.H);
      const float4* wp = reinterpret_cast<const float4*>(wbase + (size_t)h * a.N + n0);
      const float4* bp = reinterpret_cast<const float4*>(bbase + ((size_t)h * a.R + r) * a.N + n0);
#pragma unroll
      for (int q = 0; q < E / 4; ++q) {
        const float4 wv = wp[q], bv = bp[q];
        w[u][4 * q] = wv.x; w[u][4 * q + 1] = wv.y; w[u][4 * q + 2] = wv.z; w[u][4 * q + 3] = wv.w;
        b[u][4 * q] = bv.x; b[u][4 * q + 1] = bv.y; b[u][4 * q + 2] = bv.z; b[u][4 * q + 3] = bv.w;
      }
    }
    float v[kU][E], ss[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      unpack16(raw[u], v[u], (const T*)nullptr);
      ss[u] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) ss[u] = __builtin_fmaf(v[u][e], v[u][e], ss[u]);
    }
    // every lane takes part (out-of-range lanes with zeros); groups never
    // straddle rows
    for (int off = cpr >> 1; off > 0; off >>= 1)
#pragma unroll
      for (int u = 0; u < kU; ++u) ss[u] += __shfl_xor(ss[u], off, cpr);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t i = i0 + u * stride;
      if (i < nvec) {
        const float scale = 1.f / sqrtf(ss[u] / (float)a.N + a.eps);
#pragma unroll
        for (int e = 0; e < E; ++e) v[u][e] = __builtin_fmaf(v[u][e] * scale, w[u][e], b[u][e]);
        dst[i] = pack16(v[u], (const T*)nullptr);
      }
    }
  } else {
    // up-projection of 16-byte pieces of x into R pieces of X
    const int cpr = a.P / E;
    const size_t nvec = a.rows * (size_t)cpr;
    const uint4* src = static_cast<const uint4*>(a.x);
    uint4* dst = static_cast<uint4*>(a.x_out);
    uint4 raw[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t i = i0 + u * stride;
      raw[u] = i < nvec ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t i = i0 + u * stride;
      if (i >= nvec) break;
      const size_t row = i / cpr;  // (token, head)
      const int p0 = (int)(i % cpr) * E;
      const int h = (int)(row % a.H);
      float v[E];
      unpack16(raw[u], v, (const T*)nullptr);
      for (int r = 0; r < a.R; ++r) {
        const float4* up = reinterpret_cast<const float4*>(a.up + ((size_t)h * a.R + r) * a.P + p0);
        float o[E];
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
          const float4 uv = up[q];
          o[4 * q] = v[4 * q] * uv.x;
          o[4 * q + 1] = v[4 * q + 1] * uv.y;
          o[4 * q + 2] = v[4 * q + 2] * uv.z;
          o[4 * q + 3] = v[4 * q + 3] * uv.w;
        }
        dst[(row * a.R + r) * cpr + (i % cpr)] = pack16(o, (const T*)nullptr);
      }
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(kBlkThreads) postpass_kernel(BlockArgs a) {
  constexpr int E = Vec16<T>::E;
  constexpr int kRMax = 4;
  const size_t stride = (size_t)gridDim.x * kBlkThreads;
  const size_t i0 = (size_t)blockIdx.x * kBlkThreads + threadIdx.x;
  const int cpr = a.P / E;
  const size_t nvec = a.rows * (size_t)cpr;
  const uint4* src = static_cast<const uint4*>(a.y);
  uint4 raw[kU][kRMax];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const size_t i = i0 + u * stride;
    const size_t row = i / cpr;
#pragma unroll
    for (int r = 0; r < kRMax; ++r)
      raw[u][r] = (i < nvec && r < a.R) ? src[(row * a.R + r) * cpr + (i % cpr)]
                                        : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const size_t i = i0 + u * stride;
    if (i >= nvec) break;
    const size_t row = i / cpr;  // (token, head)
    const int p0 = (int)(i % cpr) * E;
    const int h = (int)(row % a.H);
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
    for (int r = 0; r < kRMax; ++r) {
      if (r >= a.R) break;
      float v[E];
      unpack16(raw[u][r], v, (const T*)nullptr);
      const float4* d = reinterpret_cast<const float4*>(a.down + ((size_t)h * a.R + r) * a.P + p0);
#pragma unroll
      for (int q = 0; q < E / 4; ++q) {
        const float4 dv = d[q];
        acc[4 * q] = __builtin_fmaf(v[4 * q], dv.x, acc[4 * q]);
        acc[4 * q + 1] = __builtin_fmaf(v[4 * q + 1], dv.y, acc[4 * q + 1]);
        acc[4 * q + 2] = __builtin_fmaf(v[4 * q + 2], dv.z, acc[4 * q + 2]);
        acc[4 * q + 3] = __builtin_fmaf(v[4 * q + 3], dv.w, acc[4 * q + 3]);
      }
    }
    static_cast<uint4*>(a.y_out)[i] = pack16(acc, (const T*)nullptr);
  }
}

dim3 grid_for(size_t nvec, unsigned parts) {
  const size_t per_block = (size_t)kBlkThreads * kU;
  return dim3((unsigned)((nvec + per_block - 1) / per_block), parts);
}

}  // namespace

hipError_t launch_block_prepass(const BlockArgs& a, m3_dtype dtype, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const size_t es = dtype == M3_BF16 ? 2 : 4, E = 16 / es;
  const size_t nbc = a.rows * a.R * (a.N / E), nx = a.rows * (a.P / E);
  const dim3 grid = grid_for(nbc > nx ? nbc : nx, 3);
  if (dtype == M3_BF16)
    hipLaunchKernelGGL(prepass_kernel<bf16>, grid, dim3(kBlkThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(prepass_kernel<float>, grid, dim3(kBlkThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_block_postpass(const BlockArgs& a, m3_dtype dtype, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const size_t es = dtype == M3_BF16 ? 2 : 4, E = 16 / es;
  const dim3 grid = grid_for(a.rows * (a.P / E), 1);
  if (dtype == M3_BF16)
    hipLaunchKernelGGL(postpass_kernel<bf16>, grid, dim3(kBlkThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(postpass_kernel<float>, grid, dim3(kBlkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace m3
