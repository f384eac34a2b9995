// decode.hip -- one fused Mamba-3 decode step on gfx950.
//
//   h' = alpha R (h + (1-lam) dt B_prev x_prev^T) + lam dt B_t x_t^T,   y = C_t^T h'
//
// (exponential-trapezoidal rule with the complex transition as 2x2 rotations;
// MIMO rank-R products.)  The step is bound by HBM traffic: each (sequence,
// head) unit reads and writes its N x P float state once, and everything else
// it touches is small (x, B, C, angles: a few KB).  So one block owns one unit:
//
//   * every thread first issues all its loads (coalesced float4 state rows,
//     its x pieces, its pair of the small inputs, kept raw), then the block
//     builds per-row coefficient vectors in LDS:
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

// Raw storage of 4 consecutive elements (an x row piece) and of a rotation
// pair, converted to float only where used.
template <typename T>
struct Raw;
template <>
struct Raw<float> {
  typedef float4 x4;
  typedef float2 pair;
};
template <>
struct Raw<bf16> {
  typedef uint2 x4;
  typedef uint32_t pair;
};
__device__ __forceinline__ float4 cvt4(float4 v) { return v; }
__device__ __forceinline__ float4 cvt4(uint2 v) {
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
}
__device__ __forceinline__ float2 cvt2(float2 v) { return v; }
__device__ __forceinline__ float2 cvt2(uint32_t v) {
  return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
}

// Everything one block reads for one unit (sequence, head): this thread's
// state rows, its x pieces, and the rotation pair it prepares coefficients
// for (thread kp < N/2), as loaded.
template <typename T, int R, int NPT>
struct DecStage {
  float4 h0[NPT], h1[NPT];
  typename Raw<T>::x4 xc[R], xq[R];
  typename Raw<T>::pair bt[R], ct[R], bp[R];
  float th, d, la, A;
};

template <typename T, int R, bool kTrap, bool kRot, int NPT>
__device__ __forceinline__ void load_stage(const DecodeArgs& a, int unit,
                                           DecStage<T, R, NPT>& st) {
  const int N = a.N, P = a.P, npair = N / 2;
  const int tid = threadIdx.x, cols4 = P / 4, c4 = tid % cols4, rg = tid / cols4;
  const int rowgroups = kDecThreads / cols4;
  const float* hin = a.h_in + (size_t)unit * N * P;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int kp = rg + i * rowgroups;
    if (kp < npair) {
      st.h0[i] = *reinterpret_cast<const float4*>(hin + (size_t)(2 * kp) * P + 4 * c4);
      st.h1[i] = *reinterpret_cast<const float4*>(hin + (size_t)(2 * kp + 1) * P + 4 * c4);
    }
  }
  typedef typename Raw<T>::x4 X4;
  typedef typename Raw<T>::pair PR;
  const T* xt = static_cast<const T*>(a.x_t) + (size_t)unit * R * P;
  const T* xp = static_cast<const T*>(a.x_prev) + (size_t)unit * R * P;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    st.xc[r] = *reinterpret_cast<const X4*>(xt + r * P + 4 * c4);
    if constexpr (kTrap) st.xq[r] = *reinterpret_cast<const X4*>(xp + r * P + 4 * c4);
  }
  const int kp = tid;
  if (kp < npair) {
    const T* Bt = static_cast<const T*>(a.B_t) + (size_t)unit * R * N;
    const T* Ct = static_cast<const T*>(a.C_t) + (size_t)unit * R * N;
    const T* Bp = static_cast<const T*>(a.B_prev) + (size_t)unit * R * N;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      st.bt[r] = *reinterpret_cast<const PR*>(Bt + r * N + 2 * kp);
      st.ct[r] = *reinterpret_cast<const PR*>(Ct + r * N + 2 * kp);
      if constexpr (kTrap) st.bp[r] = *reinterpret_cast<const PR*>(Bp + r * N + 2 * kp);
    }
    if constexpr (kRot) st.th = a.theta[(size_t)unit * npair + kp];
  }
  st.d = a.dt[unit];
  st.la = kTrap ? a.lam[unit] : 1.f;
  st.A = a.A[unit % a.H];
}

// One unit from its stage: per-row coefficients into LDS, the state update
// (stored), y through an LDS reduction over the row groups.
template <typename T, int R, bool kTrap, bool kRot, int NPT>
__device__ __forceinline__ void decode_unit(const DecodeArgs& a, int unit,
                                            const DecStage<T, R, NPT>& st, float* dsm) {
  const int N = a.N, P = a.P, npair = N / 2;
  const int tid = threadIdx.x, cols4 = P / 4, c4 = tid % cols4, rg = tid / cols4;
  const int rowgroups = kDecThreads / cols4;
  float2* s_rot = reinterpret_cast<float2*>(dsm);
  float* s_u = dsm + 2 * npair;
  float* s_v = s_u + R * N;
  float* s_c = s_v + R * N;
  float* s_y = s_c + R * N;  // [rowgroups][R][P]
  const float d = st.d, la = st.la;
  const float alpha = expf(d * st.A);
  const float cu = alpha * (1.f - la) * d, cv = la * d;
  if (tid < npair) {
    const int kp = tid;
    float sn = 0.f, cn = 1.f;
    if constexpr (kRot) sincosf(d * st.th, &sn, &cn);
    s_rot[kp] = make_float2(cn, sn);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float2 bt = cvt2(st.bt[r]), ct = cvt2(st.ct[r]);
      if constexpr (kTrap) {
        const float2 bp = cvt2(st.bp[r]);
        *reinterpret_cast<float2*>(s_u + r * N + 2 * kp) =
            make_float2(cu * (cn * bp.x - sn * bp.y), cu * (sn * bp.x + cn * bp.y));
      }
      *reinterpret_cast<float2*>(s_v + r * N + 2 * kp) = make_float2(cv * bt.x, cv * bt.y);
      *reinterpret_cast<float2*>(s_c + r * N + 2 * kp) = ct;
    }
  }
  __syncthreads();

  float4 xc[R], xq[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    xc[r] = cvt4(st.xc[r]);
    if constexpr (kTrap) xq[r] = cvt4(st.xq[r]);
  }
  float yp[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) yp[r][e] = 0.f;
  float* hout = a.h_out + (size_t)unit * N * P;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int kp = rg + i * rowgroups;
    if (kp < npair) {
      const float2 rc = s_rot[kp];
      float u0[R], u1[R], v0[R], v1[R], q0[R], q1[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if constexpr (kTrap) {
          const float2 u = *reinterpret_cast<const float2*>(s_u + r * N + 2 * kp);
          u0[r] = u.x;
          u1[r] = u.y;
        }
        const float2 v = *reinterpret_cast<const float2*>(s_v + r * N + 2 * kp);
        const float2 q = *reinterpret_cast<const float2*>(s_c + r * N + 2 * kp);
        v0[r] = v.x;
        v1[r] = v.y;
        q0[r] = q.x;
        q1[r] = q.y;
      }
      float o0[4], o1[4];
      const float a0v[4] = {st.h0[i].x, st.h0[i].y, st.h0[i].z, st.h0[i].w};
      const float a1v[4] = {st.h1[i].x, st.h1[i].y, st.h1[i].z, st.h1[i].w};
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

  // y: reduce the row groups' partials
#pragma unroll
  for (int r = 0; r < R; ++r)
    *reinterpret_cast<float4*>(s_y + (rg * R + r) * P + 4 * c4) =
        make_float4(yp[r][0], yp[r][1], yp[r][2], yp[r][3]);
  __syncthreads();
  T* y = static_cast<T*>(a.y) + (size_t)unit * R * P;
  for (int o = tid; o < R * P; o += kDecThreads) {
    float sum = 0.f;
    for (int g2 = 0; g2 < rowgroups; ++g2) sum += s_y[g2 * R * P + o];
    y[o] = from_f32<T>(sum);
  }
}

// One block per unit: its loads are all issued before any arithmetic; the
// pairs per thread are a compile-time count, so the state takes no more
// registers than the shape needs and more blocks stay resident per CU
// (their loads in flight cover each other's arithmetic).
template <typename T, int R, bool kTrap, bool kRot, int NPT>
__global__ void __launch_bounds__(kDecThreads) decode_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) float dsm[];
  DecStage<T, R, NPT> st;
  load_stage<T, R, kTrap, kRot, NPT>(a, blockIdx.x, st);
  decode_unit<T, R, kTrap, kRot, NPT>(a, blockIdx.x, st, dsm);
}

template <typename T, int R, bool kTrap, bool kRot, int NPT>
hipError_t launch_decode_npt(const DecodeArgs& a, hipStream_t stream) {
  const int rowgroups = kDecThreads / (a.P / 4);
  const size_t lds = sizeof(float) * (2 * (a.N / 2) + 3 * R * a.N + (size_t)rowgroups * R * a.P);
  const void* k = reinterpret_cast<const void*>(&decode_kernel<T, R, kTrap, kRot, NPT>);
  hipError_t e = lds_limit(k, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_kernel<T, R, kTrap, kRot, NPT>), dim3(a.S * a.H), dim3(kDecThreads),
                     lds, stream, a);
  return hipGetLastError();
}

// Pairs per thread: N/2 pairs over 256 / (P / 4) row groups.
template <typename T, int R, bool kTrap, bool kRot>
hipError_t launch_decode_mode(const DecodeArgs& a, hipStream_t stream) {
  const int npt = (a.N / 2 + kDecThreads / (a.P / 4) - 1) / (kDecThreads / (a.P / 4));
  if (npt <= 2) return launch_decode_npt<T, R, kTrap, kRot, 2>(a, stream);
  if (npt <= 4) return launch_decode_npt<T, R, kTrap, kRot, 4>(a, stream);
  return launch_decode_npt<T, R, kTrap, kRot, kMaxPairsPerThread>(a, stream);
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
