// m3_internal.h -- host-side interface between the C ABI (m3ssm_api.hip) and
// the kernel launchers.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "m3ssm.h"

namespace m3 {

constexpr int kThreads = 256;     // threads per block of every prefill kernel
constexpr int kLMax = 128;        // largest chunk (tokens)
constexpr int kLRMax = 256;       // largest chunk * R (rows of a chunk tile)
constexpr size_t kLdsLimit = 160 * 1024;  // LDS per workgroup on gfx950

// Shape of one prefill problem plus device pointers (all validated).
struct PrefillArgs {
  int nb, T, H, P, N, R, L, nC;
  const void* x;
  const float* dt;
  const float* A;
  const float* lam;
  const float* theta;
  const void* B;
  const void* C;
  void* y;
  float* h_final;
  // workspace carve
  float* S;       // [B*H][nC][P][N] chunk-local states (float)
  void* G;        // [B*H][nC][P][N] chunk entry states (storage type)
  float* decay;   // [B*H][nC]       exp of the chunk's summed log-decay
  float2* rot;    // [B*H][nC][N/2]  (cos, sin) of the chunk's summed angle
};

struct DecodeArgs {
  int S, H, P, N, R;
  const float* h_in;
  float* h_out;
  const void *x_t, *x_prev, *B_t, *B_prev, *C_t;
  const float *dt, *A, *lam, *theta;
  void* y;
};

// LDS layout of one chunk tile, identical on host and device.
struct ChunkLayout {
  int LR;      // rows of the chunk tile (tokens * R)
  int LRpad;   // LR rounded up to 32
  int ldN;     // leading dim of [rows][N] tiles (elements)
  int ldK;     // leading dim of [cols][LRpad] tiles (elements)
  uint32_t off_scal, off_part, off_a, off_b, off_xt, total;  // byte offsets
};

__host__ __device__ inline uint32_t align_up_u32(uint32_t v, uint32_t a) {
  return (v + a - 1) / a * a;
}

// out_kernel: tiles C~ [LRpad][ldN] (off_a), B~ [LRpad][ldN] (off_b), X^T [P][ldK].
// state kernel: (B~ * coef)^T [N][ldK] (off_a), X^T [P][ldK]; off_b unused.
__host__ __device__ inline ChunkLayout chunk_layout(int L, int R, int N, int P, int esize,
                                                    bool out_kernel) {
  ChunkLayout c;
  c.LR = L * R;
  c.LRpad = (c.LR + 31) / 32 * 32;
  const int pad = 16 / esize;
  c.ldN = N + pad;
  c.ldK = c.LRpad + pad;
  uint32_t o = 0;
  c.off_scal = o;
  o += 4 * kLMax * 4;
  c.off_part = o;
  o += 2 * kThreads * 4;
  c.off_a = o;
  if (out_kernel) {
    o = align_up_u32(o + (uint32_t)c.LRpad * c.ldN * esize, 16);
    c.off_b = o;
    o = align_up_u32(o + (uint32_t)c.LRpad * c.ldN * esize, 16);
  } else {
    o = align_up_u32(o + (uint32_t)N * c.ldK * esize, 16);
    c.off_b = o;
  }
  c.off_xt = o;
  o = align_up_u32(o + (uint32_t)P * c.ldK * esize, 16);
  c.total = o;
  return c;
}

hipError_t launch_prefill(const PrefillArgs& a, m3_dtype dtype, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, m3_dtype dtype, hipStream_t stream);

// Largest N the decode kernel handles for a given P.
int decode_max_n(int P);

}  // namespace m3
