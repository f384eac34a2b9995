// m3_internal.h -- host-side interface between the C ABI (m3ssm_api.hip) and
// the kernel launchers.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "m3ssm.h"

namespace m3 {

constexpr int kThreads = 512;     // threads per prefill workgroup (8 waves)
constexpr int kLMax = 128;        // largest chunk (tokens)
constexpr int kLRMax = 256;       // largest chunk * R (rows of a chunk tile)
constexpr size_t kLdsLimit = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int kMaxStTiles = 4;    // 16x16 state tiles per wave (N * P <= 8192)
constexpr int kMaxSeg = 16;       // tokens per thread in the per-pair angle scan

// Shape of one prefill problem plus device pointers (all validated).
struct PrefillArgs {
  int nb, T, H, P, N, R, L, nC;
  int K;     // chunks per segment (one workgroup walks one segment)
  int nSeg;  // segments per sequence
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
  float* ring;   // [B*H][2][N][P] exit states of the two most recent segments
  int* flags;    // [B*H] segments of each sequence whose exit state is published
  int* ticket;   // [1]   next segment ticket (work order)
  int* err;      // [1]   nonzero if a wait for a predecessor timed out
};

struct DecodeArgs {
  int S, H, P, N, R;
  const float* h_in;
  float* h_out;
  const void *x_t, *x_prev, *B_t, *B_prev, *C_t;
  const float *dt, *A, *lam, *theta;
  void* y;
};

__host__ __device__ inline uint32_t align_up_u32(uint32_t v, uint32_t a) {
  return (v + a - 1) / a * a;
}

// LDS layout of the prefill workgroup, identical on host and device.
struct ChunkLayout {
  int LR;      // rows of the chunk tile (tokens * R)
  int LRpad;   // LR rounded up to 32
  int ldN;     // leading dim of [rows][N] tiles and of the [P][N] state copy
  int ldK;     // leading dim of the [P][LRpad] X^T tile
  // byte offsets
  uint32_t off_dtr, off_lamr, off_cs, off_gam, off_om, off_dt, off_w;  // per-token floats
  uint32_t off_part;     // kThreads doubles: per-segment angle sums
  uint32_t off_crot;     // N/2 float2: (cos, sin) of the chunk's total angle
  uint32_t off_srot;     // N/2 float2: (cos, sin) of the segment's total angle
  uint32_t off_sang;     // N/2 doubles: segment angle sums
  uint32_t off_th;       // [L][N/2] floats: theta of the chunk
  uint32_t off_C, off_B; // [LRpad][ldN] C~ and B~
  uint32_t off_XT;       // [P][ldK] X^T
  uint32_t off_G;        // [P][ldN] state copy for the inter-chunk term
  uint32_t total;
};

__host__ __device__ inline ChunkLayout chunk_layout(int L, int R, int N, int P, int esize) {
  ChunkLayout c;
  c.LR = L * R;
  c.LRpad = (c.LR + 31) / 32 * 32;
  const int pad = 16 / esize;
  c.ldN = N + pad;
  c.ldK = c.LRpad + pad;
  uint32_t o = 0;
  const uint32_t tokf = (kLMax + 4) * 4;
  c.off_dtr = o; o += tokf;
  c.off_lamr = o; o += tokf;
  c.off_cs = o; o += tokf;
  c.off_gam = o; o += tokf;
  c.off_om = o; o += tokf;
  c.off_dt = o; o += tokf;
  c.off_w = o; o += tokf;
  c.off_part = o; o += kThreads * 8;
  c.off_crot = o; o += (uint32_t)(N / 2) * 8;
  c.off_srot = o; o += (uint32_t)(N / 2) * 8;
  c.off_sang = o; o += (uint32_t)(N / 2) * 8;
  o = align_up_u32(o, 16);
  c.off_th = o; o = align_up_u32(o + (uint32_t)L * (N / 2) * 4, 16);
  c.off_C = o; o = align_up_u32(o + (uint32_t)c.LRpad * c.ldN * esize, 16);
  c.off_B = o; o = align_up_u32(o + (uint32_t)c.LRpad * c.ldN * esize, 16);
  c.off_XT = o; o = align_up_u32(o + (uint32_t)P * c.ldK * esize, 16);
  c.off_G = o; o = align_up_u32(o + (uint32_t)P * c.ldN * esize, 16);
  c.total = o;
  return c;
}

// 16-byte vectors per thread needed to stage the largest input tile of a
// chunk (B/C, x or theta).
__host__ __device__ inline int chunk_stage_vectors(int L, int R, int N, int P, int esize) {
  const int vecN = L * R * N * esize / 16, vecP = L * R * P * esize / 16;
  const int vecTh = L * (N / 2) * 4 / 16;
  int m = vecN > vecP ? vecN : vecP;
  m = m > vecTh ? m : vecTh;
  return (m + kThreads - 1) / kThreads;
}

// Shapes the prefill kernel handles: staging of at most four vectors per
// thread per tile, at most four state tiles per wave, rows of whole 16-byte
// vectors that evenly divide the workgroup.
__host__ __device__ inline bool chunk_fits_registers(int L, int R, int N, int P, int esize) {
  const int vprN = N * esize / 16, vprP = P * esize / 16, vprT = N / 8;
  const int seglen = (L + kThreads / (N / 2) - 1) / (kThreads / (N / 2));
  return chunk_stage_vectors(L, R, N, P, esize) <= 4 && seglen <= kMaxSeg &&
         (N / 16) * (P / 16) <= kMaxStTiles * (kThreads / 64) && (N / 2) % 4 == 0 &&
         kThreads % vprN == 0 && kThreads % vprP == 0 && kThreads % vprT == 0;
}

hipError_t launch_prefill(const PrefillArgs& a, m3_dtype dtype, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, m3_dtype dtype, hipStream_t stream);

// Largest N the decode kernel handles for a given P.
int decode_max_n(int P);

// Chunks per segment (one prefill workgroup walks one segment).
int prefill_segment_chunks(int nb, int H, int nC);

}  // namespace m3
