// decode_mfma.hip -- the Mamba-3 decode step with the MIMO update's rank-2R
// product on the matrix cores (the same step as decode.hip, whose vector
// kernel is the default; this one is kept as a measured alternative).  Its
// own translation unit, compiled with the default instruction scheduler.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

// The same step with the update h' = alpha Rot(h) + [U V] [x_prev; x_t]
// written as one product of K = 2R: per 16 x 16 tile of h'^T (rows p, columns
// n), v_mfma_f32_16x16x4_f32 takes A = [x_prev | x_t] (16 p x 4 ranks), B =
// [U | V]^T (4 ranks x 16 n) and the accumulator C = alpha Rot(h)^T, R / 2
// products per tile.  Lane l then holds h[n][p..p+3] with n = n0 + l % 16 and
// p = p0 + 4 (l / 16), one float4 of a state row in and out.  The rotation
// partner row n ^ 1 is the neighbouring lane (a DPP swap).  y = C^T h' is
// each lane's sum over its rows, then a reduce-scatter over the 16 lanes of
// a DPP row.  Shapes: R in {2, 4}, P = 64 (one 16-column block of p per wave),
// N a multiple of 16 up to 128.
constexpr int kMfmaWaves = 4;
constexpr int kMfmaMaxNt = 8;  // 16-row tiles of n per wave

template <typename T, int R, bool kTrap, bool kRot>
__global__ void __launch_bounds__(kMfmaWaves * 64) decode_mfma_kernel(DecodeArgs a) {
  static_assert(R == 2 || R == 4, "the product takes K = 2R in steps of 4");
  extern __shared__ __align__(16) float dsm[];
  const int unit = blockIdx.x, N = a.N, npair = N / 2, nt_n = N / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int p0 = 16 * wave;
  // loads first: this lane's state pieces, its x values for the A operand
  const float* hin = a.h_in + (size_t)unit * N * 64;
  float4 hv[kMfmaMaxNt];
#pragma unroll
  for (int t = 0; t < kMfmaMaxNt; ++t)
    if (t < nt_n)
      hv[t] = *reinterpret_cast<const float4*>(hin + (size_t)(16 * t + col) * 64 + p0 + 4 * grp);
  const T* xt = static_cast<const T*>(a.x_t) + (size_t)unit * R * 64;
  const T* xp = static_cast<const T*>(a.x_prev) + (size_t)unit * R * 64;
  // A operand of product q: rank k = 4q + grp of [x_prev | x_t] at p0 + col
  float av[R / 2];
#pragma unroll
  for (int q = 0; q < R / 2; ++q) {
    const int k = 4 * q + grp;
    if (k < R)
      av[q] = kTrap ? to_f32(xp[k * 64 + p0 + col]) : 0.f;
    else
      av[q] = to_f32(xt[(k - R) * 64 + p0 + col]);
  }
  // per-row coefficients, as in the vector kernel: rotation, U, V, C
  float2* s_rot = reinterpret_cast<float2*>(dsm);
  float* s_u = dsm + 2 * npair;
  float* s_v = s_u + R * N;
  float* s_c = s_v + R * N;
  const float d = a.dt[unit], la = kTrap ? a.lam[unit] : 1.f;
  const float alpha = expf(d * a.A[unit % a.H]);
  const float cu = alpha * (1.f - la) * d, cv = la * d;
  for (int kp = tid; kp < npair; kp += kMfmaWaves * 64) {
    float sn = 0.f, cn = 1.f;
    if constexpr (kRot) sincosf(d * a.theta[(size_t)unit * npair + kp], &sn, &cn);
    s_rot[kp] = make_float2(alpha * cn, alpha * sn);
    const T* Bt = static_cast<const T*>(a.B_t) + (size_t)unit * R * N;
    const T* Ct = static_cast<const T*>(a.C_t) + (size_t)unit * R * N;
    const T* Bp = static_cast<const T*>(a.B_prev) + (size_t)unit * R * N;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if constexpr (kTrap) {
        const float b0 = to_f32(Bp[r * N + 2 * kp]), b1 = to_f32(Bp[r * N + 2 * kp + 1]);
        s_u[r * N + 2 * kp] = cu * (cn * b0 - sn * b1);
        s_u[r * N + 2 * kp + 1] = cu * (sn * b0 + cn * b1);
      } else {
        s_u[r * N + 2 * kp] = 0.f;
        s_u[r * N + 2 * kp + 1] = 0.f;
      }
      s_v[r * N + 2 * kp] = cv * to_f32(Bt[r * N + 2 * kp]);
      s_v[r * N + 2 * kp + 1] = cv * to_f32(Bt[r * N + 2 * kp + 1]);
      s_c[r * N + 2 * kp] = to_f32(Ct[r * N + 2 * kp]);
      s_c[r * N + 2 * kp + 1] = to_f32(Ct[r * N + 2 * kp + 1]);
    }
  }
  __syncthreads();

  float acc[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[r][i] = 0.f;
  float* hout = a.h_out + (size_t)unit * N * 64;
  const float sgn = (col & 1) ? 1.f : -1.f;  // row 2k: c h - s h'; row 2k+1: s h' + c h
#pragma unroll
  for (int t = 0; t < kMfmaMaxNt; ++t) {
    if (t >= nt_n) break;
    const int n = 16 * t + col;
    float4 c4;
    if constexpr (kRot) {
      const float2 rc = s_rot[n >> 1];
      // the partner row's values from the neighbouring lane (quad_perm 1,0,3,2)
      const float o0 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, hv[t].x), 0xb1, 0xf, 0xf, true));
      const float o1 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, hv[t].y), 0xb1, 0xf, 0xf, true));
      const float o2 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, hv[t].z), 0xb1, 0xf, 0xf, true));
      const float o3 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, hv[t].w), 0xb1, 0xf, 0xf, true));
      const float ss = sgn * rc.y;
      c4 = make_float4(rc.x * hv[t].x + ss * o0, rc.x * hv[t].y + ss * o1,
                       rc.x * hv[t].z + ss * o2, rc.x * hv[t].w + ss * o3);
    } else {
      c4 = make_float4(alpha * hv[t].x, alpha * hv[t].y, alpha * hv[t].z, alpha * hv[t].w);
    }
    typedef float f4v __attribute__((ext_vector_type(4)));
    f4v dacc = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
    for (int q = 0; q < R / 2; ++q) {
      const int k = 4 * q + grp;
      const float bv = k < R ? s_u[k * N + n] : s_v[(k - R) * N + n];
      dacc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], bv, dacc, 0, 0, 0);
    }
    *reinterpret_cast<float4*>(hout + (size_t)n * 64 + p0 + 4 * grp) =
        make_float4(dacc[0], dacc[1], dacc[2], dacc[3]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float cr = s_c[r * N + n];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[r][i] = __builtin_fmaf(cr, dacc[i], acc[r][i]);
    }
  }
  // y[r][p0 + 4 grp + i]: sum over the 16 lanes of the DPP row.  Values
  // v[4r + i]; reduce-scatter halves the vector at each step so that lane
  // col ends with entry col % (4R) (R = 2: lanes col and col + 8 alike).
  constexpr int V = 4 * R;
  float v[V];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) v[4 * r + i] = acc[r][i];
  if constexpr (V == 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] += __shfl_xor(v[j], 8, 16);
  }
#pragma unroll
  for (int m = V / 2; m >= 1; m >>= 1) {
    const bool up = (col & m) != 0;
#pragma unroll
    for (int j = 0; j < m; ++j) {
      const float send = up ? v[j] : v[j + m];
      const float keep = up ? v[j + m] : v[j];
      v[j] = keep + __shfl_xor(send, m, 16);
    }
  }
  const int e = col % V, r = e / 4, i = e % 4;
  if (col < V) {
    T* y = static_cast<T*>(a.y) + (size_t)unit * R * 64;
    y[r * 64 + p0 + 4 * grp + i] = from_f32<T>(v[0]);
  }
}

template <typename T, int R, bool kTrap, bool kRot>
hipError_t launch_decode_mfma_mode(const DecodeArgs& a, hipStream_t stream) {
  const size_t lds = sizeof(float) * (2 * (a.N / 2) + 3 * R * a.N);
  const void* k = reinterpret_cast<const void*>(&decode_mfma_kernel<T, R, kTrap, kRot>);
  hipError_t e = lds_limit(k, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_mfma_kernel<T, R, kTrap, kRot>), dim3(a.S * a.H),
                     dim3(kMfmaWaves * 64), lds, stream, a);
  return hipGetLastError();
}

template <typename T, int R>
hipError_t launch_decode_mfma_typed(const DecodeArgs& a, hipStream_t stream) {
  if (a.lam)
    return a.theta ? launch_decode_mfma_mode<T, R, true, true>(a, stream)
                   : launch_decode_mfma_mode<T, R, true, false>(a, stream);
  return a.theta ? launch_decode_mfma_mode<T, R, false, true>(a, stream)
                 : launch_decode_mfma_mode<T, R, false, false>(a, stream);
}

}  // namespace

bool decode_mfma_shape(int R, int N, int P) {
  return (R == 2 || R == 4) && P == 64 && N % 16 == 0 && N >= 16 && N <= 16 * kMfmaMaxNt;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, m3_dtype dtype, hipStream_t stream) {
  if (a.S == 0) return hipSuccess;
  if (!decode_mfma_shape(a.R, a.N, a.P)) return hipErrorInvalidValue;
  const bool bf = dtype == M3_BF16;
  if (a.R == 2)
    return bf ? launch_decode_mfma_typed<bf16, 2>(a, stream) : launch_decode_mfma_typed<float, 2>(a, stream);
  return bf ? launch_decode_mfma_typed<bf16, 4>(a, stream) : launch_decode_mfma_typed<float, 4>(a, stream);
}

}  // namespace m3
