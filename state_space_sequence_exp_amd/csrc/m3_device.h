// m3_device.h -- device-side building blocks shared by the libm3ssm kernels
// (gfx950 / CDNA4 only): storage types, conversions, 16x16 MFMA fragments,
// fast sine/cosine and wave-level scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m3 {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 raw bytes as a native vector (HIP's uint4 is a class; copies of it can
// keep values out of registers)
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

// Two adjacent storage elements (a rotation pair) as floats.
__device__ __forceinline__ float2 load_pair(const float* p) {
  return *reinterpret_cast<const float2*>(p);
}
__device__ __forceinline__ float2 load_pair(const bf16* p) {
  bf16x2 v = *reinterpret_cast<const bf16x2*>(p);
  return make_float2(static_cast<float>(v.x), static_cast<float>(v.y));
}

constexpr float kInv2Pi = 0.15915494309189535f;
// 2*pi split in two floats (Cody-Waite): kTwoPiHi is the float nearest 2*pi.
constexpr float kTwoPiHi = 6.28318548202514648f;
constexpr float kTwoPiLo = -1.7484555314695172e-7f;

// a + b reduced to about [-pi, pi].  Running angles are kept reduced at every
// step so that they never grow (a float near 100 rad has a 7.6e-6 ulp) and the
// reduction itself adds no systematic error.
__device__ __forceinline__ float angle_add(float a, float b) {
#pragma clang fp contract(off)
  float s = a + b;
  const float k = __builtin_rintf(s * kInv2Pi);
  s = __builtin_fmaf(-k, kTwoPiHi, s);
  return __builtin_fmaf(-k, kTwoPiLo, s);
}

// sin and cos of an angle already reduced to about [-pi, pi], on the hardware
// sine/cosine (which take revolutions).
__device__ __forceinline__ void fast_sincos(float a, float* s, float* c) {
  const float r = a * kInv2Pi;
  *s = __builtin_amdgcn_sinf(r);
  *c = __builtin_amdgcn_cosf(r);
}

// A DPP lane move of a float (lanes whose source is outside the row, or
// whose row is masked off, read 0).
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xf, false));
}

// Inclusive prefix sum across the 64 lanes of a wave, in DPP steps: shifts by
// 1, 2, 4 and 8 within each row of 16 lanes, then the last lane of row 0 (and
// of row 2) added to row 1 (row 3), then the last lane of row 1 added to rows
// 2 and 3.
__device__ __forceinline__ float wave_incl_scan(float v) {
  v += dpp_move<0x111>(v);        // row_shr:1
  v += dpp_move<0x112>(v);        // row_shr:2
  v += dpp_move<0x114>(v);        // row_shr:4
  v += dpp_move<0x118>(v);        // row_shr:8
  v += dpp_move<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_move<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// The value of lane l + 1, and `last` in lane 63 (DPP wave_shl:1; the lane
// without a source keeps the old value).  No lane condition is involved, so
// the move always runs on the whole wave (a DPP move reading a disabled lane
// would return the old value instead).
__device__ __forceinline__ float wave_next_lane(float v, float last) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(last), __float_as_int(v), 0x130, 0xf, 0xf, false));
}

// Value of lane `lane` (uniform) broadcast to the wave.
__device__ __forceinline__ float wave_read_lane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// ---------------------------------------------------------------------------
// 16x16 MFMA tiles.  Lane l holds, for A (16 x K, row-major in LDS) row l%16
// and K-slots [g*KPL, g*KPL+KPL) with g = l/16; for B (K x 16) column l%16
// and the same K-slots; the 16x16 fp32 result holds rows 4g..4g+3 of column
// l%16 (element j = row 4g+j).
template <typename T>
struct Mfma;

template <>
struct Mfma<bf16> {
  static constexpr int KPL = 8;
  static constexpr int K = 32;
  typedef bf16x8 frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // Fragment from a row-major matrix: row `row`, K-slots starting at k0.
  __device__ __forceinline__ static frag load(const bf16* base, int ld, int row, int k0) {
    const int g = (threadIdx.x & 63) >> 4;
    return *reinterpret_cast<const bf16x8*>(base + (size_t)row * ld + k0 + g * KPL);
  }
};

template <>
struct Mfma<float> {
  static constexpr int KPL = 1;
  static constexpr int K = 4;
  typedef float frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const float* base, int ld, int row, int k0) {
    const int g = (threadIdx.x & 63) >> 4;
    return base[(size_t)row * ld + k0 + g];
  }
};

}  // namespace m3
