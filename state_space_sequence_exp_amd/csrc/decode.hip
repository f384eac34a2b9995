// decode.hip -- one fused Mamba-3 decode step on gfx950.
//
//   h' = alpha R (h + (1-lam) dt B_prev x_prev^T) + lam dt B_t x_t^T,   y = C_t^T h'
//
// (exponential-trapezoidal rule with the complex transition as 2x2 rotations;
// MIMO rank-R products.)  The step is bound by HBM traffic: each (sequence,
// head) unit reads and writes its N x P float state once, and everything else
// it touches is small (x, B, C, angles: a few KB).  So one block owns one unit:
//
//   * every thread first issues its state loads (coalesced float4 rows, all in
//     flight at once), then the block builds per-row coefficient vectors in LDS:
//       rot[k]   = (cos, sin)(dt theta_k)
//       u_r[n]   = alpha (1-lam) dt (R B_prev[r])[n]
//       v_r[n]   = lam dt B_t[r][n]
//       c_r[n]   = C_t[r][n]
//   * each element then needs one 2x2 rotation, 2R fused multiply-adds and R
//     more for its share of y; y is reduced over N through LDS.
//
// Two reduced forms are compiled separately: without lam (lam = 1, the
// exponential-Euler rule of Mamba-2) the previous token's term vanishes and
// x_prev, B_prev are not read; without theta the state is real (no
// rotation) and theta is not read.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

constexpr int kDecThreads = 256;
constexpr int kMaxPairsPerThread = 8;

__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}

template <typename T, int R, bool kTrap, bool kRot>
__global__ void __launch_bounds__(kDecThreads) decode_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) float dsm[];
  const int unit = blockIdx.x;  // s * H + h
  const int hh = unit % a.H;
  const int N = a.N, P = a.P, npair = N / 2;
  const int tid = threadIdx.x;
  const int cols4 = P / 4;
  const int c4 = tid % cols4, rg = tid / cols4;
  const int rowgroups = kDecThreads / cols4;

  // 1. state loads first (all independent)
  const float* hin = a.h_in + (size_t)unit * N * P;
  float4 h0[kMaxPairsPerThread], h1[kMaxPairsPerThread];
#pragma unroll
  for (int i = 0; i < kMaxPairsPerThread; ++i) {
    const int kp = rg + i * rowgroups;
    if (kp < npair) {
      h0[i] = load4(hin + (size_t)(2 * kp) * P + 4 * c4);
      h1[i] = load4(hin + (size_t)(2 * kp + 1) * P + 4 * c4);
    }
  }
  const T* xt = static_cast<const T*>(a.x_t) + (size_t)unit * R * P;
  float4 xc[R], xq[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    xc[r] = load4(xt + r * P + 4 * c4);
    if constexpr (kTrap) {
      const T* xp = static_cast<const T*>(a.x_prev) + (size_t)unit * R * P;
      xq[r] = load4(xp + r * P + 4 * c4);
    }
  }

  // 2. per-row coefficients in LDS
  float2* s_rot = reinterpret_cast<float2*>(dsm);
  float* s_u = dsm + 2 * npair;
  float* s_v = s_u + R * N;
  float* s_c = s_v + R * N;
  float* s_y = s_c + R * N;  // [rowgroups][R][P]
  const float d = a.dt[unit], la = kTrap ? a.lam[unit] : 1.f;
  const float alpha = expf(d * a.A[hh]);
  const float cu = alpha * (1.f - la) * d, cv = la * d;
  const T* Bp = static_cast<const T*>(a.B_prev) + (size_t)unit * R * N;
  const T* Bt = static_cast<const T*>(a.B_t) + (size_t)unit * R * N;
  const T* Ct = static_cast<const T*>(a.C_t) + (size_t)unit * R * N;
  for (int kp = tid; kp < npair; kp += kDecThreads) {
    float sn = 0.f, cn = 1.f;
    if constexpr (kRot) sincosf(d * a.theta[(size_t)unit * npair + kp], &sn, &cn);
    s_rot[kp] = make_float2(cn, sn);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float2 bt = load_pair(Bt + r * N + 2 * kp);
      const float2 ct = load_pair(Ct + r * N + 2 * kp);
      if constexpr (kTrap) {
        const float2 bp = load_pair(Bp + r * N + 2 * kp);
        s_u[r * N + 2 * kp] = cu * (cn * bp.x - sn * bp.y);
        s_u[r * N + 2 * kp + 1] = cu * (sn * bp.x + cn * bp.y);
      }
      s_v[r * N + 2 * kp] = cv * bt.x;
      s_v[r * N + 2 * kp + 1] = cv * bt.y;
      s_c[r * N + 2 * kp] = ct.x;
      s_c[r * N + 2 * kp + 1] = ct.y;
    }
  }
  __syncthreads();

  // 3. update the state, accumulate y partials
  float yp[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) yp[r][e] = 0.f;
  float* hout = a.h_out + (size_t)unit * N * P;
#pragma unroll
  for (int i = 0; i < kMaxPairsPerThread; ++i) {
    const int kp = rg + i * rowgroups;
    if (kp < npair) {
      const float2 rc = s_rot[kp];
      float u0[R], u1[R], v0[R], v1[R], q0[R], q1[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if constexpr (kTrap) {
          u0[r] = s_u[r * N + 2 * kp];
          u1[r] = s_u[r * N + 2 * kp + 1];
        }
        v0[r] = s_v[r * N + 2 * kp];
        v1[r] = s_v[r * N + 2 * kp + 1];
        q0[r] = s_c[r * N + 2 * kp];
        q1[r] = s_c[r * N + 2 * kp + 1];
      }
      float o0[4], o1[4];
      const float a0v[4] = {h0[i].x, h0[i].y, h0[i].z, h0[i].w};
      const float a1v[4] = {h1[i].x, h1[i].y, h1[i].z, h1[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float n0, n1;
        if constexpr (kRot) {
          n0 = alpha * (rc.x * a0v[e] - rc.y * a1v[e]);
          n1 = alpha * (rc.y * a0v[e] + rc.x * a1v[e]);
        } else {
          n0 = alpha * a0v[e];
          n1 = alpha * a1v[e];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float xce = (&xc[r].x)[e];
          if constexpr (kTrap) {
            const float xqe = (&xq[r].x)[e];
            n0 += u0[r] * xqe + v0[r] * xce;
            n1 += u1[r] * xqe + v1[r] * xce;
          } else {
            n0 += v0[r] * xce;
            n1 += v1[r] * xce;
          }
        }
        o0[e] = n0;
        o1[e] = n1;
#pragma unroll
        for (int r = 0; r < R; ++r) yp[r][e] += q0[r] * n0 + q1[r] * n1;
      }
      *reinterpret_cast<float4*>(hout + (size_t)(2 * kp) * P + 4 * c4) =
          make_float4(o0[0], o0[1], o0[2], o0[3]);
      *reinterpret_cast<float4*>(hout + (size_t)(2 * kp + 1) * P + 4 * c4) =
          make_float4(o1[0], o1[1], o1[2], o1[3]);
    }
  }

  // 4. reduce y over row groups
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_y[(rg * R + r) * P + 4 * c4 + e] = yp[r][e];
  __syncthreads();
  T* y = static_cast<T*>(a.y) + (size_t)unit * R * P;
  for (int o = tid; o < R * P; o += kDecThreads) {
    float s = 0.f;
    for (int g2 = 0; g2 < rowgroups; ++g2) s += s_y[g2 * R * P + o];
    y[o] = from_f32<T>(s);
  }
}

template <typename T, int R, bool kTrap, bool kRot>
hipError_t launch_decode_mode(const DecodeArgs& a, hipStream_t stream) {
  const int rowgroups = kDecThreads / (a.P / 4);
  const size_t lds = sizeof(float) * (2 * (a.N / 2) + 3 * R * a.N + (size_t)rowgroups * R * a.P);
  const void* k = reinterpret_cast<const void*>(&decode_kernel<T, R, kTrap, kRot>);
  hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_kernel<T, R, kTrap, kRot>), dim3(a.S * a.H), dim3(kDecThreads), lds,
                     stream, a);
  return hipGetLastError();
}

// The mode follows the optional inputs: lam (trapezoid weight) and theta
// (rotation) may each be absent.
template <typename T, int R>
hipError_t launch_decode_typed(const DecodeArgs& a, hipStream_t stream) {
  if (a.lam)
    return a.theta ? launch_decode_mode<T, R, true, true>(a, stream)
                   : launch_decode_mode<T, R, true, false>(a, stream);
  return a.theta ? launch_decode_mode<T, R, false, true>(a, stream)
                 : launch_decode_mode<T, R, false, false>(a, stream);
}

}  // namespace

// Largest N supported by the decode kernel for a given P.
int decode_max_n(int P) { return 2 * kMaxPairsPerThread * (kDecThreads / (P / 4)); }

hipError_t launch_decode(const DecodeArgs& a, m3_dtype dtype, hipStream_t stream) {
  if (a.S == 0) return hipSuccess;
  const bool bf = dtype == M3_BF16;
  switch (a.R) {
    case 1: return bf ? launch_decode_typed<bf16, 1>(a, stream) : launch_decode_typed<float, 1>(a, stream);
    case 2: return bf ? launch_decode_typed<bf16, 2>(a, stream) : launch_decode_typed<float, 2>(a, stream);
    case 4: return bf ? launch_decode_typed<bf16, 4>(a, stream) : launch_decode_typed<float, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace m3
