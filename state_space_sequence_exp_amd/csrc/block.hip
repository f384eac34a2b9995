// block.hip -- the block-side steps on either side of the SSM (Mamba-3 paper
// translation, section 3.4; the reading of the projections is stated in
// include/m3ssm.h):
//
//   pre-pass   B~ = RMSNorm_N(B) * wB[h] + bB[h,r],  C~ likewise   (BCNorm + bias)
//              X[r] = x * U[h,r]                                   (MIMO up-projection)
//   post-pass  y_out = sum_r D[h,r] * y[r]                         (MIMO down-projection)
//
// Both passes stream their operands once and are bound by HBM bandwidth, so
// they are laid out for coalescing rather than for the matrix cores.  Each
// tensor is seen as [token][M] 16-byte vectors (8 bfloat16 or 4 float; M the
// vectors of one token, over all heads and ranks); thread j owns column
// m = j % M of the kU consecutive tokens of group j / M, issuing all their
// loads first.  So consecutive lanes move consecutive vectors, a workgroup
// touches a few contiguous runs (one per token of its group), and a thread's
// weights, which depend on the column only, are read once.  The pre-pass is
// one launch over three row spaces (blockIdx.y: B rows, C rows, x rows); a B
// or C row of N channels is N / E consecutive lanes (E elements per vector,
// N / E a power of two dividing the wave), whose sum of squares is reduced by
// lane shuffles inside that group.
#include <algorithm>
#include <initializer_list>

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

// Tokens per thread (its column's vectors in kU consecutive tokens).
constexpr int kU = 8;

// Thread j of a row space of M columns and `ntok` tokens: its column and its
// first token (ntok or beyond: the thread has nothing to do).
struct Slot {
  size_t m, t0;
};
__device__ __forceinline__ Slot slot_of(size_t M, int u_per) {
  const size_t j = (size_t)blockIdx.x * kBlkThreads + threadIdx.x;
  return Slot{j % M, (j / M) * (size_t)u_per};
}

template <int E>
__device__ __forceinline__ void load_w(const float* p, float (&w)[E]) {
#pragma unroll
  for (int q = 0; q < E / 4; ++q) {
    const float4 v = reinterpret_cast<const float4*>(p)[q];
    w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
  }
}

template <typename T>
__global__ void __launch_bounds__(kBlkThreads) prepass_kernel(BlockArgs a) {
  constexpr int E = Vec16<T>::E;
  const size_t ntok = a.rows / a.H;
  const int part = blockIdx.y;
  if (part < 2) {
    // BCNorm + bias on 16-byte pieces of B or C rows
    const int cpr = a.N / E;  // lanes per row: a power of two that divides the wave
    const size_t M = (size_t)a.H * a.R * cpr;
    const Slot sl = slot_of(M, kU);
    // a lane group of one row shares its token group, so whole groups leave
    if (sl.t0 >= ntok) return;
    const uint4* src = static_cast<const uint4*>(part == 0 ? a.B : a.C);
    uint4* dst = static_cast<uint4*>(part == 0 ? a.B_out : a.C_out);
    uint4 raw[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t t = sl.t0 + u;
      raw[u] = t < ntok ? src[t * M + sl.m] : make_uint4(0u, 0u, 0u, 0u);
    }
    // column m is piece m % cpr of rank (m / cpr) % R of head m / (cpr R)
    const int n0 = (int)(sl.m % cpr) * E, r = (int)((sl.m / cpr) % a.R);
    const int h = (int)(sl.m / ((size_t)cpr * a.R));
    float w[E], b[E];
    load_w<E>((part == 0 ? a.norm_B : a.norm_C) + (size_t)h * a.N + n0, w);
    load_w<E>((part == 0 ? a.bias_B : a.bias_C) + ((size_t)h * a.R + r) * a.N + n0, b);
    float v[kU][E], ss[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      unpack16(raw[u], v[u], (const T*)nullptr);
      ss[u] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) ss[u] = __builtin_fmaf(v[u][e], v[u][e], ss[u]);
    }
    // every lane of a group takes part (tokens past the end with zeros)
    for (int off = cpr >> 1; off > 0; off >>= 1)
#pragma unroll
      for (int u = 0; u < kU; ++u) ss[u] += __shfl_xor(ss[u], off, cpr);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t t = sl.t0 + u;
      if (t < ntok) {
        const float scale = 1.f / sqrtf(ss[u] / (float)a.N + a.eps);
#pragma unroll
        for (int e = 0; e < E; ++e) v[u][e] = __builtin_fmaf(v[u][e] * scale, w[e], b[e]);
        dst[t * M + sl.m] = pack16(v[u], (const T*)nullptr);
      }
    }
  } else {
    // up-projection of 16-byte pieces of x into R pieces of X
    constexpr int kRMax = 4;
    const int cpr = a.P / E;
    const size_t M = (size_t)a.H * cpr;
    const Slot sl = slot_of(M, kU);
    if (sl.t0 >= ntok) return;
    const uint4* src = static_cast<const uint4*>(a.x);
    uint4* dst = static_cast<uint4*>(a.x_out);
    uint4 raw[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t t = sl.t0 + u;
      raw[u] = t < ntok ? src[t * M + sl.m] : make_uint4(0u, 0u, 0u, 0u);
    }
    // column m is piece c of head h; X row (token, head) holds R pieces per
    // column, rank-major
    const int c = (int)(sl.m % cpr), p0 = c * E, h = (int)(sl.m / cpr);
    float up[kRMax][E];
#pragma unroll
    for (int r = 0; r < kRMax; ++r)
      if (r < a.R) load_w<E>(a.up + ((size_t)h * a.R + r) * a.P + p0, up[r]);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t t = sl.t0 + u;
      if (t >= ntok) break;
      const size_t row = t * a.H + h;  // (token, head)
      float v[E];
      unpack16(raw[u], v, (const T*)nullptr);
#pragma unroll
      for (int r = 0; r < kRMax; ++r) {
        if (r >= a.R) break;
        float o[E];
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = v[e] * up[r][e];
        dst[(row * a.R + r) * cpr + c] = pack16(o, (const T*)nullptr);
      }
    }
  }
}

// The post-pass reads R pieces per output piece: R is a template argument
// (registers), and with R = 4 a thread takes half as many pieces.
template <int R>
constexpr int post_pieces() {
  return R == 4 ? kU / 2 : kU;
}

template <typename T, int R>
__global__ void __launch_bounds__(kBlkThreads) postpass_kernel(BlockArgs a) {
  constexpr int E = Vec16<T>::E;
  constexpr int U = post_pieces<R>();
  const size_t ntok = a.rows / a.H;
  const int cpr = a.P / E;
  const size_t M = (size_t)a.H * cpr;  // output pieces per token
  const Slot sl = slot_of(M, U);
  if (sl.t0 >= ntok) return;
  const int c = (int)(sl.m % cpr), p0 = c * E, h = (int)(sl.m / cpr);
  const uint4* src = static_cast<const uint4*>(a.y);
  uint4 raw[U][R];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t t = sl.t0 + u;
    const size_t row = t * a.H + h;  // (token, head)
#pragma unroll
    for (int r = 0; r < R; ++r)
      raw[u][r] = t < ntok ? src[(row * R + r) * cpr + c] : make_uint4(0u, 0u, 0u, 0u);
  }
  float dw[R][E];
#pragma unroll
  for (int r = 0; r < R; ++r) load_w<E>(a.down + ((size_t)h * R + r) * a.P + p0, dw[r]);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t t = sl.t0 + u;
    if (t >= ntok) break;
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float v[E];
      unpack16(raw[u][r], v, (const T*)nullptr);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(v[e], dw[r][e], acc[e]);
    }
    static_cast<uint4*>(a.y_out)[t * M + sl.m] = pack16(acc, (const T*)nullptr);
  }
}

// Blocks for the threads of row spaces of M columns over ntok tokens, u
// tokens per thread: M times the token groups, the widest space.
dim3 grid_for(size_t ntok, int u, unsigned parts, std::initializer_list<size_t> widths) {
  size_t threads = 0;
  for (size_t M : widths) {
    const size_t t = M * ((ntok + u - 1) / u);
    if (t > threads) threads = t;
  }
  return dim3((unsigned)std::min<size_t>((threads + kBlkThreads - 1) / kBlkThreads, 0xffffffffu),
              parts);
}

}  // namespace

hipError_t launch_block_prepass(const BlockArgs& a, m3_dtype dtype, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const size_t es = dtype == M3_BF16 ? 2 : 4, E = 16 / es;
  const dim3 grid = grid_for(a.rows / a.H, kU, 3,
                             {(size_t)a.H * a.R * (a.N / E), (size_t)a.H * (a.P / E)});
  if (grid.x > 0x7fffffffu) return hipErrorInvalidValue;
  if (dtype == M3_BF16)
    hipLaunchKernelGGL(prepass_kernel<bf16>, grid, dim3(kBlkThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(prepass_kernel<float>, grid, dim3(kBlkThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int R>
hipError_t launch_post(const BlockArgs& a, hipStream_t stream) {
  constexpr size_t E = Vec16<T>::E;
  const dim3 grid = grid_for(a.rows / a.H, post_pieces<R>(), 1, {(size_t)a.H * (a.P / E)});
  if (grid.x > 0x7fffffffu) return hipErrorInvalidValue;
  hipLaunchKernelGGL((postpass_kernel<T, R>), grid, dim3(kBlkThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_post_t(const BlockArgs& a, hipStream_t stream) {
  switch (a.R) {
    case 1: return launch_post<T, 1>(a, stream);
    case 2: return launch_post<T, 2>(a, stream);
    case 4: return launch_post<T, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_block_postpass(const BlockArgs& a, m3_dtype dtype, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  return dtype == M3_BF16 ? launch_post_t<bf16>(a, stream) : launch_post_t<float>(a, stream);
}

}  // namespace m3
