// prefill_impl.h -- the fused chunked prefill kernel of the Mamba-3
// recurrence on gfx950, templated on storage type, MIMO rank and head
// dimension.  Included by one translation unit per storage type.
//
// The sequence of each (batch b, head h) is cut into chunks of L tokens and
// the chunks into segments of K chunks.  One workgroup (512 threads, one per
// CU) owns one segment and runs three phases:
//
//  1. Local pass.  For each chunk: per-token log-decay prefix sums cs_u,
//     trapezoid weights gamma_u = lam_u dt_u and omega_u = (1 - lam_{u+1})
//     dt_{u+1}, chunk-local cumulative angles phi_u[k] (per rotation pair),
//     rotated inputs B~_u = R(phi_u)^T B_u (the data-dependent RoPE of
//     Proposition 3, Mamba-3 paper summary), the chunk state
//     S_c = sum_u exp(cs_e - cs_u)(gamma_u + omega_u) B~_u x_u^T on MFMA, and
//     the chunk-level recurrence G <- R(Phi_c)(exp(cs_e) G + S_c) from G = 0.
//     The result is the segment's exit state for a zero entry state, plus the
//     segment's total decay and total angle.
//  2. Chain.  Wait for the exit state of the previous segment of the same
//     sequence, combine (the recurrence is linear: E_exit = R(Phi)(D E_entry)
//     + E_local), publish this segment's exit state.
//  3. Output pass.  Walk the chunks again from the true entry state:
//         y_t = exp(cs_t) C~_t^T G_c
//             + sum_{u<=t} exp(cs_t - cs_u)(gamma_u + [u<t] omega_u)(C~_t^T B~_u) x_u^T
//     i.e. the chunk's structured mask (decay matrix x 2-band trapezoid
//     matrix; Mamba-3 paper translation, section 3.1, equation 7) applied to
//     C~ B~^T on MFMA, plus the inter-chunk term, then the same chunk-level
//     recurrence to the next chunk.
//
// Frames.  Angles restart at every chunk, so the entry state G_c of a chunk
// is in the unrotated (API) frame, and the previous token's trapezoid term
// omega B x^T is folded into it: G_c = h_{cL-1} + omega_{cL-1} B_{cL-1}
// x_{cL-1}^T.  No halo token is needed inside a chunk.  Running angles inside
// a chunk are kept in revolutions, reduced to [0, 1) at every token (the
// hardware sine takes revolutions); chunk and segment totals are summed in
// double and take the accurate sine/cosine, since the chain multiplies their
// rotations over the whole sequence.
//
// One chunk step, per workgroup:
//   [P] every thread sums dt*theta over its rotation item (one rotation pair,
//       S consecutive tokens) from registers staged a chunk ahead; wave 0
//       computes the per-token scalars.                          -- barrier
//   [R] every thread finishes its item's angles from the other items' sums,
//       rotates its B (and C) pairs and writes B~, C~ and the weighted,
//       transposed B~ into LDS; x goes to LDS transposed; the next chunk's
//       inputs are requested.                                     -- barrier
//   [F] MFMA: outputs (phase 3) and the chunk state, folded into the state
//       tiles held in registers.
// The per-token scalars alternate between two LDS buffers, so [P] of the next
// chunk does not wait for [F] of this one.
//
// Memory.  Inputs are read with buffer loads whose range ends at the last
// valid byte of the chunk's sequence, so rows past the end of a sequence
// read as zero and y rows past it are dropped by the buffer store.  The five
// chunk tiles live unpadded in LDS with each 16-byte column XOR-swizzled by
// row, so the MFMA fragment reads (16 lanes on 16 rows of one column) hit
// distinct banks.
//
// Work order and the chain.  Workgroups take tickets from a counter; ticket
// t is segment t / (B*H) of sequence t % (B*H).  A workgroup only waits for a
// smaller ticket, which is held by a running workgroup, so the grid always
// drains.  Segments publish their aggregate (the map from entry to exit
// state) or their exit state in a per-ticket slot with device-coherent (sc1)
// stores and loads, and a per-ticket status word that is raised only after
// the stores have completed; a segment finds its entry by looking back over
// its predecessors' slots (in groups, see phase 2).  Every wait is bounded
// and raises an error word (1) instead of hanging.  A ticket outside the grid
// (counters not zero at entry) raises the error word (2) and does no work.
#pragma once

#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace pf {

constexpr int kT = kPrefillThreads;
constexpr int kW = kT / kWave;             // waves per workgroup
constexpr int kSpinLimit = 1 << 18;        // bounded wait (a few hundred ms)
constexpr int kGroup = 8;                  // segments per look-back group
constexpr int kBatch = 4;                  // aggregates loaded at once in the look-back
constexpr int kRsrcWord3 = 0x00020000;     // raw buffer descriptor, gfx9 family
constexpr uint32_t kOOB = 0x7ff00000u;     // a buffer offset past every range
constexpr double kInv2PiD = 0.15915494309189533577;

typedef __amdgpu_buffer_rsrc_t rsrc;

// A uniform value the compiler treats as unknown from here on.  Applied at the
// top of every chunk step to the strides and LDS offsets that per-thread
// addresses derive from, so those addresses are recomputed in each step (a
// few VALU) instead of being hoisted out of the chunk loops and kept in
// registers for the whole kernel, which would spill.
__device__ __forceinline__ uint32_t opaque_u(uint32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}
__device__ __forceinline__ uint32_t ld32(rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x2 ld64(rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2 v = {from_f32<bf16>(lo), from_f32<bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// A [rows][row_bytes] tile in LDS.  For 2-byte types its 16-byte columns are
// XOR-swizzled by row within aligned groups of up to eight columns (128
// bytes), so the 16 rows an MFMA fragment read touches spread over all banks.
// An offset that is a multiple of 128 bytes still adds straight to an
// address, so fragment addresses are one of two per-lane bases (for the two
// halves of a 128-byte group) plus an immediate.  4-byte tiles are not
// swizzled.
struct Tile {
  unsigned char* base;
  uint32_t rowb, mask;
  __device__ __forceinline__ uint32_t at(uint32_t row, uint32_t byte) const {
    return row * rowb + ((((byte >> 4) ^ (row & mask)) << 4) | (byte & 15u));
  }
  template <typename V>
  __device__ __forceinline__ V& ref(uint32_t row, uint32_t byte) const {
    return *reinterpret_cast<V*>(base + at(row, byte));
  }
  // element at byte `byte` of the row, split as (byte mod 128) through the
  // swizzle and (byte - byte mod 128) added afterwards
  template <typename V>
  __device__ __forceinline__ const V& ref2(uint32_t row, uint32_t lane_byte,
                                           uint32_t group_byte) const {
    const uint32_t b = lane_byte + group_byte;
    return *reinterpret_cast<const V*>(base + at(row, b & 127u) + (b & ~127u));
  }
};
__device__ __forceinline__ Tile make_tile(unsigned char* base, uint32_t rowb, int esize) {
  const uint32_t ncol = rowb >> 4;
  const uint32_t low = ncol & (0u - ncol);
  return Tile{base, rowb, esize == 2 ? (low < 8u ? low : 8u) - 1u : 0u};
}

template <typename T_, int R_, int P_, int N_>
struct Cfg {
  using T = T_;
  using M = Mfma<T_>;
  static constexpr int R = R_, P = P_;
  static constexpr int NC = N_;  // state size if fixed at compile time, else 0
  // aggregates loaded at once in the chain's look-back (fewer with more
  // state per wave: registers)
  static constexpr int kAggBatch = N_ == 64 ? kBatch : (N_ != 0 ? kBatch / 2 : 1);
  static constexpr int es = (int)sizeof(T_);
  static constexpr int S = prefill_item_tokens(es, R_, N_, P_);  // tokens per rotation item
  static constexpr int KR = S * R_;                      // chunk rows per item
  static constexpr int PW = es / 2;                      // 32-bit words per pair
  static constexpr int NPT = P_ / 16;                    // p-tiles
  // N = 64 fixed, P <= 64, R = 1: at most four output units, so the output
  // pass keeps the state tiles on the other four waves only, and the state
  // update runs beside the outputs (the local pass spreads them over all)
  static constexpr bool kSplit3 = N_ == 64 && P_ <= 64 && R_ == 1 && kPrefillThreads == 512;
  // the output pass's score hand-over may apply (prefill_score_handover
  // decides with the chunk length)
  static constexpr bool kHand3 = sizeof(T_) == 2 && prefill_score_handover(64, R_, N_, P_, true);
  // sixteen query blocks a chunk (chunk R = 256, so R >= 2) may take the
  // uneven dealing of chunk_output
  static constexpr bool kDeal16 = R_ >= 2 && kPrefillThreads == 512;
  // N fixed with N / 2 pairs dividing the wave: wave w holds token blocks
  // w * 128 / N .. (w + 1) * 128 / N - 1 of every pair, and the angle sums
  // before a block are the wave totals of the waves before it plus, with two
  // blocks per wave, the lower half's sum (see step_partials)
  static constexpr bool kWaveSums = N_ != 0 && 64 % (N_ / 2) == 0 && 64 / (N_ / 2) <= 2;
};

// Raw inputs of one chunk for this thread, staged in registers.  With wave
// sums every lane of a wave has its tokens among the wave's 64 / (N / 2)
// blocks, so the wave loads those tokens' dt once (lane j: the wave's token
// j, in dtw) and each lane takes its own when they are used (stage_dt).
template <class C>
struct Stage {
  float th[C::S], dt[C::S];                                  // rotation item
  uint32_t dtw;
  uint32_t b[C::KR * C::PW], c[C::KR * C::PW], x[C::KR * C::PW];
};

// This thread's dt of its rotation item's tokens.
template <class C>
__device__ __forceinline__ void stage_dt(const Stage<C>& st, float (&dt)[C::S]) {
  if constexpr (C::kWaveSums) {
    // lanes 32..63 hold the wave's second block when there are two
    constexpr int kBlocks = 64 / (C::NC / 2);
    const bool upper = kBlocks == 2 && (threadIdx.x & 32) != 0;
#pragma unroll
    for (int j = 0; j < C::S; ++j) {
      const float lo = __uint_as_float(__builtin_amdgcn_readlane(st.dtw, j));
      if constexpr (kBlocks == 2) {
        const float hi = __uint_as_float(__builtin_amdgcn_readlane(st.dtw, C::S + j));
        dt[j] = upper ? hi : lo;
      } else {
        dt[j] = lo;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < C::S; ++j) dt[j] = st.dt[j];
  }
}

// The wave that computes the per-token scalars of the next chunk during the
// MFMA phase (it holds no output unit when the outputs fit in few waves).
constexpr int kScalarWave = kW - 1;

// Uniform per-workgroup values.
struct Ctx {
  int b, h, bh, seg, c0, c1;
  uint32_t rowB, rowTh, rowDt, rowX;  // token strides in bytes
  float Ah;
};

// This thread's rotation item (pair kp, token block blk) and x item (column
// pair jp, token block xblk).
struct Map {
  int kp, blk, jp, xblk;
  bool act, xact;
  bool xwave;  // some lane of this wave has an x item (uniform)
  int wblk;    // block of the wave's lane 0 (uniform)
};

struct ChunkRes {
  rsrc B, C, th, dt, x;
  int t0, len;
};

template <class C>
__device__ __forceinline__ ChunkRes chunk_res(const PrefillArgs& a, const Ctx& s, int c) {
  ChunkRes r;
  r.t0 = c * a.L;
  r.len = min(a.L, a.T - r.t0);
  const size_t hrow = ((size_t)s.b * a.T + r.t0) * a.H + s.h;  // [B,T,H] row of token t0
  const uint32_t last = (uint32_t)(r.len - 1);
  const uint32_t bcb = (uint32_t)(C::R * a.N * C::es);
  r.B = make_rsrc(static_cast<const unsigned char*>(a.B) + hrow * bcb, last * s.rowB + bcb);
  r.C = make_rsrc(static_cast<const unsigned char*>(a.C) + hrow * bcb, last * s.rowB + bcb);
  // without theta (a real state) the range is empty and every angle reads 0
  r.th = a.theta ? make_rsrc(a.theta + hrow * (a.N / 2), last * s.rowTh + (uint32_t)(a.N / 2) * 4)
                 : make_rsrc(nullptr, 0);
  r.dt = make_rsrc(a.dt + hrow, last * s.rowDt + 4);
  const uint32_t xb = (uint32_t)(C::R * C::P * C::es);
  r.x = make_rsrc(static_cast<const unsigned char*>(a.x) + hrow * xb, last * s.rowX + xb);
  return r;
}

// Rotation-item inputs (theta, dt, B and optionally C) of item (kp, blk).
template <class C, bool kWithC>
__device__ __forceinline__ void load_item(const PrefillArgs& a, const Ctx& s, const ChunkRes& r,
                                          uint32_t vB, uint32_t vTh, uint32_t vDt, uint32_t vDw,
                                          float (&th)[C::S], float (&dt)[C::S], uint32_t& dtw,
                                          uint32_t (&bv)[C::KR * C::PW],
                                          uint32_t (&cv)[C::KR * C::PW]) {
#pragma unroll
  for (int j = 0; j < C::S; ++j) th[j] = __uint_as_float(ld32(r.th, vTh + j * s.rowTh));
  if constexpr (C::kWaveSums) {
    dtw = ld32(r.dt, vDw);
  } else {
#pragma unroll
    for (int j = 0; j < C::S; ++j) dt[j] = __uint_as_float(ld32(r.dt, vDt + j * s.rowDt));
  }
#pragma unroll
  for (int j = 0; j < C::S; ++j)
#pragma unroll
    for (int q = 0; q < C::R; ++q) {
      const uint32_t o = vB + j * s.rowB + (uint32_t)(q * a.N * C::es);
      const int i = j * C::R + q;
      if constexpr (C::PW == 1) {
        bv[i] = ld32(r.B, o);
        if constexpr (kWithC) cv[i] = ld32(r.C, o);
      } else {
        const u32x2 v = ld64(r.B, o);
        bv[2 * i] = v.x;
        bv[2 * i + 1] = v.y;
        if constexpr (kWithC) {
          const u32x2 w = ld64(r.C, o);
          cv[2 * i] = w.x;
          cv[2 * i + 1] = w.y;
        }
      }
    }
}

template <class C>
__device__ __forceinline__ void load_x_item(const Ctx& s, const ChunkRes& r, uint32_t vX,
                                            uint32_t (&xv)[C::KR * C::PW]) {
#pragma unroll
  for (int j = 0; j < C::S; ++j)
#pragma unroll
    for (int q = 0; q < C::R; ++q) {
      const uint32_t o = vX + j * s.rowX + (uint32_t)(q * C::P * C::es);
      const int i = j * C::R + q;
      if constexpr (C::PW == 1) {
        xv[i] = ld32(r.x, o);
      } else {
        const u32x2 v = ld64(r.x, o);
        xv[2 * i] = v.x;
        xv[2 * i + 1] = v.y;
      }
    }
}

// Request all of this thread's inputs of chunk c.
template <class C, bool kWithC>
__device__ __forceinline__ void issue_loads(const PrefillArgs& a, const Ctx& s, const Map& m,
                                            int c, Stage<C>& st) {
  const ChunkRes r = chunk_res<C>(a, s, c);
  // chunk-relative byte offsets of this thread's items (past every range if
  // it has none, so the loads return zeros)
  const uint32_t tb = (uint32_t)(m.blk * C::S);
  const uint32_t vB = m.act ? tb * s.rowB + (uint32_t)(2 * m.kp * C::es) : kOOB;
  const uint32_t vTh = m.act ? tb * s.rowTh + (uint32_t)(m.kp * 4) : kOOB;
  const uint32_t vDt = m.act ? tb * s.rowDt : kOOB;
  const uint32_t vX = m.xact ? (uint32_t)(m.xblk * C::S) * s.rowX + (uint32_t)(2 * m.jp * C::es)
                             : kOOB;
  // wave sums: lane j loads the dt of the wave's token j (its first block's
  // first token on), for the wave's 64 / (N / 2) blocks of S tokens
  uint32_t vDw = kOOB;
  if constexpr (C::kWaveSums) {
    const uint32_t lane = threadIdx.x & 63;
    vDw = lane < (uint32_t)(64 / (C::NC / 2) * C::S) ? (m.wblk * C::S + lane) * s.rowDt : kOOB;
  }
  load_item<C, kWithC>(a, s, r, vB, vTh, vDt, vDw, st.th, st.dt, st.dtw, st.b, st.c);
  // x items are dealt from thread 0: waves past them issue no x loads
  if (m.xwave) load_x_item<C>(s, r, vX, st.x);
}

// dt and lam of tokens lane, lane + 64, lane + 128 of chunk c, up to the end
// of the sequence (the token after the chunk feeds omega of its last token).
// With NJ = 2 (chunks of at most 64 tokens) the third group is not loaded
// and reads as zero.
// With `real` false the range is empty: the loads read zeros and touch no
// memory.
template <int NJ = 3>
__device__ __forceinline__ void scalar_loads(const PrefillArgs& a, const Ctx& s, int c,
                                             float (&wd)[3], float (&wl)[3], bool real) {
  const int t0 = c * a.L;
  const size_t hrow = ((size_t)s.b * a.T + t0) * a.H + s.h;
  // the range covers the 3 * 64 tokens read at most (a range over the rest of
  // the sequence could wrap 32 bits on long sequences with many heads)
  const uint32_t bytes = real ? (uint32_t)(min(a.T - t0, 3 * kWave) - 1) * s.rowDt + 4 : 0u;
  const rsrc rw = make_rsrc(a.dt + hrow, bytes);
  const rsrc rl = a.lam ? make_rsrc(a.lam + hrow, bytes) : make_rsrc(nullptr, 0);
#pragma unroll
  for (int jj = 0; jj < 3; ++jj) {
    const uint32_t o = (uint32_t)((threadIdx.x & 63) + jj * 64) * s.rowDt;
    if (jj < NJ) {
      wd[jj] = __uint_as_float(ld32(rw, o));
      // without lam the weight is 1 (the exponential-Euler rule)
      wl[jj] = a.lam ? __uint_as_float(ld32(rl, o)) : 1.f;
    } else {
      wd[jj] = 0.f;
      wl[jj] = 0.f;
    }
  }
}

// Per-token scalars of the chunk (one wave): cs (inclusive prefix of dt*A),
// gamma, gamma + omega, the state weight w_u = exp(cs_e - cs_u)(gamma_u +
// omega_u) and the chunk's log-decay cs_e.  Tokens past the sequence get
// zeros (and a flat cs).
__device__ __forceinline__ void chunk_scalars(const PrefillArgs& a, int t0, int len, float Ah,
                                              const float (&wd)[3], const float (&wl)[3],
                                              float* sc) {
  const int lane = threadIdx.x & (kWave - 1);
  float cs[2] = {0.f, 0.f}, ga[2] = {0.f, 0.f}, gom[2] = {0.f, 0.f};
  float carry = 0.f;
  const int nj = a.L > kWave ? 2 : 1;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    if (jj < nj) {
      const int u = lane + kWave * jj;
      const float d = u < len ? wd[jj] : 0.f;
      // dt and lam of token u + 1: the next lane, or lane 0 of the next
      // group of 64 tokens for the last lane
      const float dn = wave_next_lane(wd[jj], wave_read_lane(wd[jj + 1], 0));
      const float ln = wave_next_lane(wl[jj], wave_read_lane(wl[jj + 1], 0));
      const float g = u < len ? wl[jj] * d : 0.f;
      const float om = (u < len && t0 + u + 1 < a.T) ? (1.f - ln) * dn : 0.f;
      cs[jj] = wave_incl_scan(d * Ah) + carry;
      carry = wave_read_lane(cs[jj], kWave - 1);
      ga[jj] = g;
      gom[jj] = g + om;
    }
  }
  const float cse = wave_read_lane(a.L > kWave ? cs[1] : cs[0], (a.L - 1) & (kWave - 1));
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int u = lane + kWave * jj;
    if (jj < nj && u < a.L) {
      sc[u] = cs[jj];
      sc[kLMax + u] = ga[jj];
      sc[2 * kLMax + u] = gom[jj];
      sc[3 * kLMax + u] = __expf(cse - cs[jj]) * gom[jj];
    }
  }
  if (lane == 0) sc[4 * kLMax] = cse;
}

// An angle in radians (a double sum of float angles) reduced to [-pi, pi].
__device__ __forceinline__ double reduce_angle(double x) {
  constexpr double kTwoPi = 6.283185307179586476925;
  return x - kTwoPi * __builtin_rint(x * kInv2PiD);
}

// KR values of one row of a K-major tile (BwT or XT) at byte offset kb
// (whole 16-byte pieces, or one 8-byte piece).
template <typename T, int KR>
__device__ __forceinline__ void store_krow(const Tile& t, uint32_t row, uint32_t kb,
                                           const float (&v)[KR]) {
  if constexpr (sizeof(T) == 2) {
    static_assert(KR == 4 || KR % 8 == 0, "row of 8 bytes or whole 16-byte pieces");
    if constexpr (KR == 4) {
      const u32x2 w = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      t.ref<u32x2>(row, kb) = w;
    } else {
#pragma unroll
      for (int h = 0; h < KR / 8; ++h) {
        const u32x4 w = {pack_bf16(v[8 * h], v[8 * h + 1]), pack_bf16(v[8 * h + 2], v[8 * h + 3]),
                         pack_bf16(v[8 * h + 4], v[8 * h + 5]),
                         pack_bf16(v[8 * h + 6], v[8 * h + 7])};
        t.ref<u32x4>(row, kb + 16 * h) = w;
      }
    }
  } else {
    static_assert(KR % 4 == 0, "whole 16-byte pieces");
#pragma unroll
    for (int h = 0; h < KR / 4; ++h)
      t.ref<f32x4>(row, kb + 16 * h) = f32x4{v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]};
  }
}

// Sum of dt*theta over one item's tokens, in double.
template <int S>
__device__ __forceinline__ double item_angle_sum(const float (&th)[S], const float (&dt)[S]) {
  double sum = 0.0;
#pragma unroll
  for (int j = 0; j < S; ++j) sum += static_cast<double>(dt[j] * th[j]);
  return sum;
}

// Rotation item (pair kp, token block blk): angles from the preceding blocks'
// sums, rotated B~ (and C~) pairs, the weighted transposed B~ rows, and for
// the last block the chunk's total rotation (and the segment angle sum).
// s_part holds the items' angle sums (block-major), or with wave sums the
// waves' totals (wave-major) and inw the sum of this wave's blocks before
// this one; s_crot receives the chunk's total rotation per pair and s_sang
// the segment's angle sums.
template <class C, bool kWithC, bool kAccumSeg>
__device__ __forceinline__ void rotate_item(int npair, int nblk, int kp, int blk,
                                            const float (&th)[C::S], const float (&dt)[C::S],
                                            const uint32_t (&bv)[C::KR * C::PW],
                                            const uint32_t (&cv)[C::KR * C::PW],
                                            const float* s_w, const Tile& tB, const Tile& tC,
                                            const Tile& tW, const double* s_part, double inw,
                                            float2* s_crot, double* s_sang) {
  using T = typename C::T;
  constexpr int R = C::R;
  // sum of the preceding blocks' angles
  double pre = inw;
  if constexpr (C::kWaveSums) {
    // the totals of the waves before this one, all requested at once
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    double v[kW - 1];
#pragma unroll
    for (int q = 0; q < kW - 1; ++q) v[q] = s_part[q * npair + kp];
#pragma unroll
    for (int q = 0; q < kW - 1; ++q) pre += q < wave ? v[q] : 0.0;
  } else {
#pragma unroll 8
    for (int q = 0; q < blk; ++q) pre += s_part[q * npair + kp];
  }
  double rv = pre * kInv2PiD;
  rv -= __builtin_rint(rv);
  float r = static_cast<float>(rv);  // revolutions
  float wb0[C::KR], wb1[C::KR];
  const uint32_t pb = (uint32_t)(2 * kp * C::es);  // byte column of the pair
#pragma unroll
  for (int j = 0; j < C::S; ++j) {
    const int u = blk * C::S + j;
    r = __builtin_amdgcn_fractf(__builtin_fmaf(dt[j] * th[j], kInv2Pi, r));
    const float sn = __builtin_amdgcn_sinf(r), cn = __builtin_amdgcn_cosf(r);
    const float w = s_w[u];
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int i = j * R + q;
      const uint32_t row = (uint32_t)(u * R + q);
      float b0, b1;
      if constexpr (C::PW == 1) {
        b0 = lo_bf16(bv[i]);
        b1 = hi_bf16(bv[i]);
      } else {
        b0 = __uint_as_float(bv[2 * i]);
        b1 = __uint_as_float(bv[2 * i + 1]);
      }
      const float rb0 = cn * b0 + sn * b1, rb1 = cn * b1 - sn * b0;
      wb0[i] = w * rb0;
      wb1[i] = w * rb1;
      if constexpr (kWithC) {
        float c0, c1;
        if constexpr (C::PW == 1) {
          c0 = lo_bf16(cv[i]);
          c1 = hi_bf16(cv[i]);
        } else {
          c0 = __uint_as_float(cv[2 * i]);
          c1 = __uint_as_float(cv[2 * i + 1]);
        }
        const float rc0 = cn * c0 + sn * c1, rc1 = cn * c1 - sn * c0;
        if constexpr (C::PW == 1) {
          tB.ref<uint32_t>(row, pb) = pack_bf16(rb0, rb1);
          tC.ref<uint32_t>(row, pb) = pack_bf16(rc0, rc1);
        } else {
          tB.ref<float2>(row, pb) = make_float2(rb0, rb1);
          tC.ref<float2>(row, pb) = make_float2(rc0, rc1);
        }
      }
    }
  }
  const uint32_t kb = (uint32_t)(blk * C::KR * C::es);
  store_krow<T, C::KR>(tW, (uint32_t)(2 * kp), kb, wb0);
  store_krow<T, C::KR>(tW, (uint32_t)(2 * kp + 1), kb, wb1);
  if (blk == nblk - 1) {
    // the chunk's total angle; the chain multiplies its rotation over the
    // whole sequence, so it takes the accurate sine/cosine
    const double tot = pre + item_angle_sum<C::S>(th, dt);
    float sn, cn;
    sincosf(static_cast<float>(reduce_angle(tot)), &sn, &cn);
    s_crot[kp] = make_float2(cn, sn);
    if constexpr (kAccumSeg) s_sang[kp] = reduce_angle(s_sang[kp] + tot);
  }
}

// x item (pair of columns jp, token block xb) -> two rows of X^T.
template <class C>
__device__ __forceinline__ void write_x_item(int jp, int xb, const uint32_t (&xv)[C::KR * C::PW],
                                             const Tile& tX) {
  const uint32_t kb = (uint32_t)(xb * C::KR * C::es);
  if constexpr (C::PW == 1) {
    if constexpr (C::KR == 4) {
      const u32x2 r0 = {__builtin_amdgcn_perm(xv[1], xv[0], 0x05040100u),
                        __builtin_amdgcn_perm(xv[3], xv[2], 0x05040100u)};
      const u32x2 r1 = {__builtin_amdgcn_perm(xv[1], xv[0], 0x07060302u),
                        __builtin_amdgcn_perm(xv[3], xv[2], 0x07060302u)};
      tX.ref<u32x2>((uint32_t)(2 * jp), kb) = r0;
      tX.ref<u32x2>((uint32_t)(2 * jp + 1), kb) = r1;
    } else {
      static_assert(C::KR % 8 == 0, "x item of 4 rows or whole 8-row pieces");
#pragma unroll
      for (int h = 0; h < C::KR / 8; ++h) {
        u32x4 r0, r1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          r0[i] = __builtin_amdgcn_perm(xv[8 * h + 2 * i + 1], xv[8 * h + 2 * i], 0x05040100u);
          r1[i] = __builtin_amdgcn_perm(xv[8 * h + 2 * i + 1], xv[8 * h + 2 * i], 0x07060302u);
        }
        tX.ref<u32x4>((uint32_t)(2 * jp), kb + 16 * h) = r0;
        tX.ref<u32x4>((uint32_t)(2 * jp + 1), kb + 16 * h) = r1;
      }
    }
  } else {
    static_assert(C::KR % 4 == 0, "fp32 x item of whole 4-row pieces");
#pragma unroll
    for (int h = 0; h < C::KR / 4; ++h) {
      tX.ref<u32x4>((uint32_t)(2 * jp), kb + 16 * h) =
          u32x4{xv[8 * h], xv[8 * h + 2], xv[8 * h + 4], xv[8 * h + 6]};
      tX.ref<u32x4>((uint32_t)(2 * jp + 1), kb + 16 * h) =
          u32x4{xv[8 * h + 1], xv[8 * h + 3], xv[8 * h + 5], xv[8 * h + 7]};
    }
  }
}

// MFMA fragment of a tile: row `row`, contraction slots from k0 (a multiple
// of 32 for bf16).
__device__ __forceinline__ bf16x8 load_frag(const Tile& t, uint32_t row, int k0, const bf16*) {
  const int g = (threadIdx.x & 63) >> 4;
  return t.ref2<bf16x8>(row, 16u * g, (uint32_t)k0 * 2u);
}
__device__ __forceinline__ float load_frag(const Tile& t, uint32_t row, int k0, const float*) {
  const int g = (threadIdx.x & 63) >> 4;
  return t.ref2<float>(row, 4u * g, (uint32_t)k0 * 4u);
}

// State tile slot m of this wave: tile index i (n-tile i % (N/16), p-tile
// i / (N/16)), or -1.  Tiles go to the state waves [sw0, sw0 + nsw) round
// robin; lane holds rows n = 4g..4g+3 of its 16x16 tile.
__device__ __forceinline__ int state_tile(const WaveRoles& wr, int wave, int m, int ntiles) {
  const int i = (wave - wr.sw0) + m * wr.nsw;
  return (wave >= wr.sw0 && wave < wr.sw0 + wr.nsw && i < ntiles) ? i : -1;
}

// State tiles -> LDS copy G^T [P][N] (the B operand of the inter-chunk MFMA).
template <class C>
__device__ __forceinline__ void state_to_lds(const PrefillArgs& a, const WaveRoles& wr,
                                             const f32x4 (&stt)[kMaxStTiles], const Tile& tG) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int ntn = a.N / 16, ntiles = ntn * C::NPT;
#pragma unroll
  for (int m = 0; m < kMaxStTiles; ++m) {
    const int i = state_tile(wr, wave, m, ntiles);
    if (i >= 0) {
      const int nt = i % ntn, pt = i / ntn;
      const uint32_t row = (uint32_t)(pt * 16 + li), nb = (uint32_t)((nt * 16 + 4 * g) * C::es);
      if constexpr (C::es == 2) {
        const u32x2 w = {pack_bf16(stt[m][0], stt[m][1]), pack_bf16(stt[m][2], stt[m][3])};
        tG.ref<u32x2>(row, nb) = w;
      } else {
        tG.ref<f32x4>(row, nb) = stt[m];
      }
    }
  }
}

// Compile-time view of a wave's state tiles when N is fixed and the tiles
// sit on the last NSW waves: with the tile count a multiple of NSW every state
// wave holds exactly kTPW tiles and no per-tile conditions are needed.
template <class C, int NSW = kW>
struct StateTiles {
  static constexpr int kNT = C::NC ? (C::NC / 16) * C::NPT : 0;
  static constexpr bool kFull = kNT != 0 && kNT % NSW == 0 && kNT / NSW <= kMaxStTiles;
  static constexpr int kTPW = kFull ? kNT / NSW : kMaxStTiles;
  static constexpr int kFirst = kW - NSW;  // first state wave
};

// Chunk state S_c = sum_u w_u B~_u x_u^T (MFMA, both operands read straight
// from the K-major tiles) folded into this wave's state tiles: st <- R(Phi_c)
// (d st + S_c).  The tiles sit on the last NSW waves (wr says the same).
template <class C, int NSW = kW>
__device__ __forceinline__ void state_update(const PrefillArgs& a, const PrefillLayout& lay,
                                             const WaveRoles& wr, float d,
                                             f32x4 (&stt)[kMaxStTiles], const Tile& tW,
                                             const Tile& tX, const unsigned char* smem) {
  using T = typename C::T;
  using M = typename C::M;
  using ST = StateTiles<C, NSW>;
  constexpr int TPW = ST::kTPW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int ntn = a.N / 16, ntiles = ntn * C::NPT;
  if (state_tile(wr, wave, 0, ntiles) < 0) return;
  const float2* s_crot = reinterpret_cast<const float2*>(smem + lay.off_crot);
  f32x4 acc[TPW];
  int tile[TPW];
  uint32_t nrow[TPW], prow[TPW];
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    tile[m] = ST::kFull ? wave - ST::kFirst + m * NSW : state_tile(wr, wave, m, ntiles);
    const int i = tile[m] < 0 ? 0 : tile[m];
    nrow[m] = (uint32_t)((i % ntn) * 16 + li);
    prow[m] = (uint32_t)((i / ntn) * 16 + li);
  }
  // a wave's tiles share their n-tile when N/16 divides the number of state
  // waves: then one A fragment serves all
  const bool share = (wr.nsw % ntn) == 0;
  if constexpr (ST::kFull && sizeof(T) == 2) {
    // N fixed: the contraction runs over the whole row of 64 R slots (the
    // rows past the chunk are zero), unrolled, with the fragments of the
    // next step requested before the MFMAs of this one
    constexpr int KS = 64 * C::R / M::K;
    typename M::frag fa[2], fb[2][TPW];
    fa[0] = load_frag(tW, nrow[0], 0, (const T*)nullptr);
#pragma unroll
    for (int m = 0; m < TPW; ++m) fb[0][m] = load_frag(tX, prow[m], 0, (const T*)nullptr);
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int cb = k & 1;
      if (k + 1 < KS) {
        fa[cb ^ 1] = load_frag(tW, nrow[0], (k + 1) * M::K, (const T*)nullptr);
#pragma unroll
        for (int m = 0; m < TPW; ++m)
          fb[cb ^ 1][m] = load_frag(tX, prow[m], (k + 1) * M::K, (const T*)nullptr);
      }
#pragma unroll
      for (int m = 0; m < TPW; ++m) {
        const typename M::frag am =
            share ? fa[cb] : load_frag(tW, nrow[m], k * M::K, (const T*)nullptr);
        acc[m] = M::mma(am, fb[cb][m], acc[m]);
      }
    }
  } else
  for (int k0 = 0; k0 < lay.LRp; k0 += M::K) {
    const typename M::frag fa0 = load_frag(tW, nrow[0], k0, (const T*)nullptr);
#pragma unroll
    for (int m = 0; m < TPW; ++m)
      if (ST::kFull || tile[m] >= 0) {
        const typename M::frag fa =
            (m == 0 || share) ? fa0 : load_frag(tW, nrow[m], k0, (const T*)nullptr);
        const typename M::frag fb = load_frag(tX, prow[m], k0, (const T*)nullptr);
        acc[m] = M::mma(fa, fb, acc[m]);
      }
  }
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    if (ST::kFull || tile[m] >= 0) {
      const int kq = (tile[m] % ntn) * 8 + 2 * g;
      const float2 r0 = s_crot[kq], r1 = s_crot[kq + 1];
      const float v0 = d * stt[m][0] + acc[m][0], v1 = d * stt[m][1] + acc[m][1];
      const float v2 = d * stt[m][2] + acc[m][2], v3 = d * stt[m][3] + acc[m][3];
      stt[m][0] = r0.x * v0 - r0.y * v1;
      stt[m][1] = r0.y * v0 + r0.x * v1;
      stt[m][2] = r1.x * v2 - r1.y * v3;
      stt[m][3] = r1.y * v2 + r1.x * v3;
    }
  }
}

// cs, gamma and gamma + omega of the tokens of chunk rows row0 .. row0+3
// (row0 a multiple of 4), as whole-vector LDS reads.
template <int R>
__device__ __forceinline__ void key_scalars4(const float* sc, int row0, float (&cs)[4],
                                             float (&ga)[4], float (&gom)[4]) {
  const float* s_cs = sc;
  const float* s_ga = sc + kLMax;
  const float* s_gom = sc + 2 * kLMax;
  if constexpr (R == 1) {
    const float4 c = *reinterpret_cast<const float4*>(s_cs + row0);
    const float4 g = *reinterpret_cast<const float4*>(s_ga + row0);
    const float4 o = *reinterpret_cast<const float4*>(s_gom + row0);
    cs[0] = c.x; cs[1] = c.y; cs[2] = c.z; cs[3] = c.w;
    ga[0] = g.x; ga[1] = g.y; ga[2] = g.z; ga[3] = g.w;
    gom[0] = o.x; gom[1] = o.y; gom[2] = o.z; gom[3] = o.w;
  } else if constexpr (R == 2) {
    const float2 c = *reinterpret_cast<const float2*>(s_cs + row0 / 2);
    const float2 g = *reinterpret_cast<const float2*>(s_ga + row0 / 2);
    const float2 o = *reinterpret_cast<const float2*>(s_gom + row0 / 2);
    cs[0] = cs[1] = c.x; cs[2] = cs[3] = c.y;
    ga[0] = ga[1] = g.x; ga[2] = ga[3] = g.y;
    gom[0] = gom[1] = o.x; gom[2] = gom[3] = o.y;
  } else {
    const float c = s_cs[row0 / 4], g = s_ga[row0 / 4], o = s_gom[row0 / 4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cs[j] = c;
      ga[j] = g;
      gom[j] = o;
    }
  }
}

// Scores of key blocks kb .. kb+KB-1 (rows) against the unit's queries
// (columns) times the chunk's mask: exp(cs_t - cs_u)(gamma_u + omega_u) for
// keys u before the query t, gamma_t on the diagonal, 0 after it.  Lane
// (g, li) holds key rows 4g .. 4g+3 of each block and query column li.
template <int R, int KB>
__device__ __forceinline__ void mask_scores(f32x4 (&sct)[KB], const float (&kcs)[KB][4],
                                            const float (&kga)[KB][4],
                                            const float (&kgom)[KB][4], int kb, int g, int tq,
                                            float csq) {
#pragma unroll
  for (int i = 0; i < KB; ++i) {
    // branch-free: every lane takes the exponential of each of its key
    // tokens (rows 4g .. 4g+3 hold 4 / R tokens; the argument is 0 for keys
    // not before the query, so it stays finite), then selects
    constexpr int TPG = R < 4 ? 4 / R : 1;
    float e[TPG];
#pragma unroll
    for (int k = 0; k < TPG; ++k) {
      const int tk = ((kb + i) * 16 + 4 * g + k * R) / R;
      e[k] = __expf(tk < tq ? csq - kcs[i][k * R] : 0.f);
      asm volatile("" : "+v"(e[k]));  // keep the exponential out of a branch
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tk = ((kb + i) * 16 + 4 * g + j) / R;
      sct[i][j] *= tk < tq ? e[j / R] * kgom[i][j] : (tk == tq ? kga[i][j] : 0.f);
    }
  }
}

// y rows of the unit (query block qb, PPG p-tiles from p_lo) to global memory.
template <class C, int PPG>
__device__ __forceinline__ void store_unit(const Ctx& s, const rsrc& ry, int qb, int p_lo,
                                           const f32x4 (&acc)[PPG]) {
  constexpr int R = C::R, P = C::P;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = qb * 16 + 4 * g + j;
    const uint32_t u = (uint32_t)(row / R), q = (uint32_t)(row % R);
    const uint32_t off = u * s.rowX + (q * P + (uint32_t)li) * C::es;
#pragma unroll
    for (int pp = 0; pp < PPG; ++pp) {
      const uint32_t o = off + (uint32_t)((p_lo + pp) * 16 * C::es);
      if constexpr (C::es == 2)
        __builtin_amdgcn_raw_buffer_store_b16(
            __builtin_bit_cast(unsigned short, from_f32<bf16>(acc[pp][j])), ry, (int)o, 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[pp][j]), ry, (int)o, 0, 0);
    }
  }
}

// The output pass's score hand-over (see prefill_score_handover): ex holds
// the handed blocks, flag counts the givers' blocks, target is the count
// that completes this chunk's (0: no hand-over).
struct ScoreX {
  uint32_t* ex;
  int* flag;
  int target;
};

// Giver: wave kW/2 + 2 i + k computes the masked scores of key block k (of
// the first pair) against query block 2 + i, as bfloat16 in the lane layout
// the taker's MFMA operand has, and counts it once its stores are done.
template <class C>
__device__ __forceinline__ void scores_give(const float* sc, const Tile& tC, const Tile& tB,
                                            const ScoreX& hx) {
  using M = typename C::M;
  constexpr int NK = C::NC / M::K;
  const int lane = threadIdx.x & 63, gw = (threadIdx.x >> 6) - kW / 2;
  const int g = lane >> 4, li = lane & 15;
  const int qx = 2 + gw / 2, kb = gw % 2;
  const int tq = qx * 16 + li;
  typename M::frag fk[NK], fq[NK];
#pragma unroll
  for (int n = 0; n < NK; ++n) {
    fk[n] = load_frag(tB, (uint32_t)(kb * 16 + li), n * M::K, (const bf16*)nullptr);
    fq[n] = load_frag(tC, (uint32_t)tq, n * M::K, (const bf16*)nullptr);
  }
  float kcs[1][4], kga[1][4], kgom[1][4];
  key_scalars4<1>(sc, kb * 16 + 4 * g, kcs[0], kga[0], kgom[0]);
  const float csq = sc[tq];
  f32x4 sct[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int n = 0; n < NK; ++n) sct[0] = M::mma(fk[n], fq[n], sct[0]);  // keys x queries
  mask_scores<1, 1>(sct, kcs, kga, kgom, kb, g, tq, csq);
  reinterpret_cast<u32x2*>(hx.ex)[gw * 64 + lane] =
      u32x2{pack_bf16(sct[0][0], sct[0][1]), pack_bf16(sct[0][2], sct[0][3])};
  // one count per wave (the release orders all of the wave's stores)
  if (lane == 0)
    __hip_atomic_fetch_add(hx.flag, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Taker: the first key pair's term of query block qb (2 or 3) from the
// handed scores.  The wait is bounded; running out (which the givers, with
// no wait of their own, cannot cause) is reported as a timed-out wait.
template <class C, int PPG>
__device__ __forceinline__ void scores_take(const PrefillArgs& a, const ScoreX& hx, int qb,
                                            int p_lo, const Tile& tX, f32x4 (&acc)[PPG]) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  bf16x4 xlo[PPG], xhi[PPG];
#pragma unroll
  for (int pp = 0; pp < PPG; ++pp) {
    const uint32_t xr = (uint32_t)((p_lo + pp) * 16 + li);
    xlo[pp] = tX.ref2<bf16x4>(xr, 8u * g, 0u);
    xhi[pp] = tX.ref2<bf16x4>(xr, 32u + 8u * g, 0u);
  }
  int spins = 0;
  while (__hip_atomic_load(hx.flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < hx.target) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > (1 << 20)) {
      __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
  }
  const u32x2 v0 = reinterpret_cast<const u32x2*>(hx.ex)[(qb - 2) * 128 + lane];
  const u32x2 v1 = reinterpret_cast<const u32x2*>(hx.ex)[(qb - 2) * 128 + 64 + lane];
  const bf16x8 fa = __builtin_bit_cast(bf16x8, u32x4{v0[0], v0[1], v1[0], v1[1]});
#pragma unroll
  for (int pp = 0; pp < PPG; ++pp) {
    bf16x8 fb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      fb[j] = xlo[pp][j];
      fb[4 + j] = xhi[pp][j];
    }
    acc[pp] = Mfma<bf16>::mma(fa, fb, acc[pp]);
  }
}

// One output unit: y rows of query block qb for the PPG p-tiles from p_lo.
// With the score hand-over query blocks 2 and 3 take their first key pair's
// scores from the givers.
template <class C, int PPG>
__device__ __forceinline__ void output_unit(const PrefillArgs& a, const Ctx& s, const rsrc& ry,
                                            int qb, int p_lo, const float* sc, const Tile& tC,
                                            const Tile& tB, const Tile& tX, const Tile& tG,
                                            const ScoreX& hx) {
  using T = typename C::T;
  using M = typename C::M;
  constexpr int R = C::R;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const int N = a.N;
  const float* s_cs = sc;
  f32x4 acc[PPG];
#pragma unroll
  for (int pp = 0; pp < PPG; ++pp) acc[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t qrow = (uint32_t)(qb * 16 + li);
  const int tq = (qb * 16 + li) / R;
  const float csq = s_cs[tq];
  constexpr int KB = (sizeof(T) == 2) ? 2 : 1;  // 16-row key blocks per step

  if constexpr (C::NC == 64) {
    // N = 64 fixed (bfloat16): the query fragments are loaded once for the
    // inter-chunk term and every key block, and each step requests all of
    // its LDS operands before its first MFMA, so their latencies overlap
    // (with N = 128 the registers for this are not there)
    constexpr int NK = C::NC / M::K;
    typename M::frag fq[NK];
#pragma unroll
    for (int n = 0; n < NK; ++n) fq[n] = load_frag(tC, qrow, n * M::K, (const T*)nullptr);
#pragma unroll
    for (int n = 0; n < NK; ++n) {
      typename M::frag fg[PPG];
#pragma unroll
      for (int pp = 0; pp < PPG; ++pp)
        fg[pp] = load_frag(tG, (uint32_t)((p_lo + pp) * 16 + li), n * M::K, (const T*)nullptr);
#pragma unroll
      for (int pp = 0; pp < PPG; ++pp) acc[pp] = M::mma(fq[n], fg[pp], acc[pp]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float scl = __expf(s_cs[(qb * 16 + 4 * g + j) / R]);
#pragma unroll
      for (int pp = 0; pp < PPG; ++pp) acc[pp][j] *= scl;
    }
    for (int kb = 0; kb * 16 <= qb * 16 + 15; kb += KB) {
      // key fragments two n-steps at a time (the next pair is requested
      // before the current pair's MFMAs)
      typename M::frag fk[KB][2];
#pragma unroll
      for (int i = 0; i < KB; ++i)
        fk[i][0] = load_frag(tB, (uint32_t)((kb + i) * 16 + li), 0, (const T*)nullptr);
      bf16x4 xlo[PPG], xhi[PPG];
#pragma unroll
      for (int pp = 0; pp < PPG; ++pp) {
        const uint32_t xr = (uint32_t)((p_lo + pp) * 16 + li);
        // key rows kb*16 + 4g.. and (kb+1)*16 + 4g..
        xlo[pp] = tX.ref2<bf16x4>(xr, 8u * g, (uint32_t)kb * 32u);
        xhi[pp] = tX.ref2<bf16x4>(xr, 32u + 8u * g, (uint32_t)kb * 32u);
      }
      float kcs[KB][4], kga[KB][4], kgom[KB][4];
#pragma unroll
      for (int i = 0; i < KB; ++i) key_scalars4<R>(sc, (kb + i) * 16 + 4 * g, kcs[i], kga[i], kgom[i]);
      f32x4 sct[KB];
#pragma unroll
      for (int i = 0; i < KB; ++i) sct[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int n = 0; n < NK; ++n) {
        if (n + 1 < NK) {
#pragma unroll
          for (int i = 0; i < KB; ++i)
            fk[i][(n + 1) & 1] =
                load_frag(tB, (uint32_t)((kb + i) * 16 + li), (n + 1) * M::K, (const T*)nullptr);
        }
#pragma unroll
        for (int i = 0; i < KB; ++i) sct[i] = M::mma(fk[i][n & 1], fq[n], sct[i]);  // keys x queries
      }
      mask_scores<R, KB>(sct, kcs, kga, kgom, kb, g, tq, csq);
      bf16x8 fa;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        fa[j] = from_f32<bf16>(sct[0][j]);
        fa[4 + j] = from_f32<bf16>(sct[1][j]);
      }
#pragma unroll
      for (int pp = 0; pp < PPG; ++pp) {
        bf16x8 fb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          fb[j] = xlo[pp][j];
          fb[4 + j] = xhi[pp][j];
        }
        acc[pp] = Mfma<bf16>::mma(fa, fb, acc[pp]);
      }
    }
  } else {
    // inter-chunk term: C~ G_c, rows scaled by exp(cs_t)
    for (int n0 = 0; n0 < N; n0 += M::K) {
      const typename M::frag fa = load_frag(tC, qrow, n0, (const T*)nullptr);
#pragma unroll
      for (int pp = 0; pp < PPG; ++pp) {
        const typename M::frag fb =
            load_frag(tG, (uint32_t)((p_lo + pp) * 16 + li), n0, (const T*)nullptr);
        acc[pp] = M::mma(fa, fb, acc[pp]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float scl = __expf(s_cs[(qb * 16 + 4 * g + j) / R]);
#pragma unroll
      for (int pp = 0; pp < PPG; ++pp) acc[pp][j] *= scl;
    }

    // intra-chunk term over key blocks up to the diagonal (from the second
    // pair where the first one's scores are handed over)
    const bool take = C::kHand3 && hx.target > 0 && qb >= 2;
    for (int kb = take ? 2 : 0; kb * 16 <= qb * 16 + 15; kb += KB) {
      // the step's x pieces and key scalars first: the mask's empty asm
      // statement keeps the scheduler from moving reads across it
      bf16x4 xlo[PPG], xhi[PPG];
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int pp = 0; pp < PPG; ++pp) {
          const uint32_t xr = (uint32_t)((p_lo + pp) * 16 + li);
          // key rows kb*16 + 4g.. and (kb+1)*16 + 4g..
          xlo[pp] = tX.ref2<bf16x4>(xr, 8u * g, (uint32_t)kb * 32u);
          xhi[pp] = tX.ref2<bf16x4>(xr, 32u + 8u * g, (uint32_t)kb * 32u);
        }
      }
      float kcs[KB][4], kga[KB][4], kgom[KB][4];
#pragma unroll
      for (int i = 0; i < KB; ++i) key_scalars4<R>(sc, (kb + i) * 16 + 4 * g, kcs[i], kga[i], kgom[i]);
      f32x4 sct[KB];
#pragma unroll
      for (int i = 0; i < KB; ++i) sct[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int n0 = 0; n0 < N; n0 += M::K) {
        const typename M::frag fq = load_frag(tC, qrow, n0, (const T*)nullptr);
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          const typename M::frag fk =
              load_frag(tB, (uint32_t)((kb + i) * 16 + li), n0, (const T*)nullptr);
          sct[i] = M::mma(fk, fq, sct[i]);  // rows = keys, cols = queries
        }
      }
      mask_scores<R, KB>(sct, kcs, kga, kgom, kb, g, tq, csq);
      if constexpr (sizeof(T) == 2) {
        bf16x8 fa;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          fa[j] = from_f32<bf16>(sct[0][j]);
          fa[4 + j] = from_f32<bf16>(sct[1][j]);
        }
#pragma unroll
        for (int pp = 0; pp < PPG; ++pp) {
          bf16x8 fb;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            fb[j] = xlo[pp][j];
            fb[4 + j] = xhi[pp][j];
          }
          acc[pp] = Mfma<bf16>::mma(fa, fb, acc[pp]);
        }
      } else {
#pragma unroll
        for (int pp = 0; pp < PPG; ++pp) {
          const f32x4 xv =
              tX.ref2<f32x4>((uint32_t)((p_lo + pp) * 16 + li), 16u * g, (uint32_t)kb * 64u);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[pp] = Mfma<float>::mma(sct[0][j], xv[j], acc[pp]);
        }
      }
    }
    if constexpr (C::kHand3)
      if (take) scores_take<C, PPG>(a, hx, qb, p_lo, tX, acc);
  }
  store_unit<C, PPG>(s, ry, qb, p_lo, acc);
}

// y of one chunk: units (query block qb, group of p-tiles) over the output
// waves.  The scores of a query block are computed once per unit, so with one
// p-group per query block nothing is recomputed.
template <class C>
__device__ __forceinline__ void chunk_output(const PrefillArgs& a, const PrefillLayout& lay,
                                             const WaveRoles& wr, const Ctx& s,
                                             const ChunkRes& cr, const float* sc, const Tile& tC,
                                             const Tile& tB, const Tile& tX, const Tile& tG,
                                             const ScoreX& hx) {
  constexpr int NPT = C::NPT;
  constexpr int PPG_A = NPT < 4 ? NPT : 4;  // the two p-group widths in use
  constexpr int PPG_B = NPT < 2 ? NPT : 2;
  const int wave = threadIdx.x >> 6;
  const size_t hrow = ((size_t)s.b * a.T + cr.t0) * a.H + s.h;
  const uint32_t yb = (uint32_t)(C::R * C::P * C::es);
  const rsrc ry = make_rsrc(static_cast<unsigned char*>(a.y) + hrow * yb,
                            (uint32_t)(cr.len - 1) * s.rowX + yb);
  if constexpr (C::kHand3) {
    // (four units on waves 0 .. kW/2-1: the others give)
    if (hx.target > 0 && wave >= kW / 2) {
      scores_give<C>(sc, tC, tB, hx);
      return;
    }
  }
  if (C::kDeal16 && wr.nout == 2 * kW && wr.npg == 1 && wr.ppg == PPG_A) {
    // sixteen query blocks, one unit each, two a wave.  Waves w and w + 4
    // share a SIMD, and the older one (w < 4) issues first, so an even split
    // leaves the younger one running alone at the end; the older wave takes
    // units of cost 13 and its partner 9 (in steps of eight MFMAs: one for
    // the inter-chunk term, one per key pair), the larger unit first.  The
    // younger waves also request the next chunk's inputs only after the
    // step's second barrier (see the output pass).
    constexpr int kDeal[8][2] = {{14, 4}, {15, 5}, {12, 6}, {13, 7},
                                 {10, 0}, {11, 1}, {8, 2}, {9, 3}};
    const int w = __builtin_amdgcn_readfirstlane(wave) & 7;
#pragma unroll
    for (int k = 0; k < 2; ++k)
      output_unit<C, PPG_A>(a, s, ry, kDeal[w][k], 0, sc, tC, tB, tX, tG, hx);
    return;
  }
  // wave w takes units w, 2kW-1-w, 2kW+w, ... so the causal (growing) cost
  // per query block balances when the units outnumber the waves
  for (int k = 0;; ++k) {
    const int unit = (k & 1) ? (k + 1) * kW - 1 - wave : k * kW + wave;
    if (unit >= wr.nout) break;
    const int qb = unit / wr.npg, p_lo = (unit % wr.npg) * wr.ppg;
    if (wr.ppg == PPG_A)
      output_unit<C, PPG_A>(a, s, ry, qb, p_lo, sc, tC, tB, tX, tG, hx);
    else
      output_unit<C, PPG_B>(a, s, ry, qb, p_lo, sc, tC, tB, tX, tG, hx);
  }
}

// Tiles of the workgroup's LDS.
struct Tiles {
  Tile C, B, W, X, G;
};

template <class C>
__device__ __forceinline__ Tiles make_tiles(const PrefillArgs& a, const PrefillLayout& lay,
                                            unsigned char* smem) {
  const uint32_t nb = (uint32_t)(a.N * C::es), kb = (uint32_t)(lay.KM * C::es);
  return Tiles{make_tile(smem + lay.off_Cr, nb, C::es), make_tile(smem + lay.off_Br, nb, C::es),
               make_tile(smem + lay.off_BwT, kb, C::es), make_tile(smem + lay.off_XT, kb, C::es),
               make_tile(smem + lay.off_GT, nb, C::es)};
}

// Per-step copies of the strides and tiles (see opaque_u).
__device__ __forceinline__ Ctx step_ctx(const Ctx& s) {
  Ctx r = s;
  r.rowB = opaque_u(s.rowB);
  r.rowTh = opaque_u(s.rowTh);
  r.rowDt = opaque_u(s.rowDt);
  r.rowX = opaque_u(s.rowX);
  return r;
}
// With N fixed the geometry is a compile-time constant (prefill_fixed_shape:
// rows of N elements, contraction-major rows of 64 R) and only the bases are
// made opaque.
template <class C>
__device__ __forceinline__ Tiles step_tiles(const Tiles& t, unsigned char* smem) {
  Tiles r;
  const Tile* src[5] = {&t.C, &t.B, &t.W, &t.X, &t.G};
  Tile* dst[5] = {&r.C, &r.B, &r.W, &r.X, &r.G};
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint32_t off = opaque_u((uint32_t)(src[i]->base - smem));
    if constexpr (C::NC != 0) {
      const bool km = i == 2 || i == 3;
      const uint32_t rowb = (uint32_t)((km ? 64 * C::R : C::NC) * C::es);
      const uint32_t ncol = rowb >> 4, low = ncol & (0u - ncol);
      *dst[i] = Tile{smem + off, rowb, (low < 8u ? low : 8u) - 1u};
    } else {
      *dst[i] = Tile{smem + off, opaque_u(src[i]->rowb), opaque_u(src[i]->mask)};
    }
  }
  return r;
}

// [P]: this thread's item's angle sum into LDS.  With wave sums (N fixed) a
// wave's total per pair goes to LDS instead, and the return value is the sum
// of this wave's blocks before this thread's (the lower half's sum for lanes
// 32..63 when a wave holds two blocks, else 0).  Items fill whole waves.
template <class C>
__device__ __forceinline__ double step_partials(const PrefillArgs& a, const PrefillLayout& lay,
                                                const Ctx& s, const Map& m, int c,
                                                const Stage<C>& st, float* sc,
                                                unsigned char* smem) {
  double* s_part = reinterpret_cast<double*>(smem + lay.off_part);
  if constexpr (C::kWaveSums) {
    if (!m.act) return 0.0;
    float dt[C::S];
    stage_dt<C>(st, dt);
    const double own = item_angle_sum<C::S>(st.th, dt);
    const int wave = threadIdx.x >> 6;
    if constexpr (C::NC / 2 == 32) {
      // lanes l and l + 32 hold blocks 2w and 2w + 1 of pair l % 32:
      // v_permlane32_swap with both operands own gives (own of lanes 0..31)
      // twice in the first result and (own of lanes 32..63) twice in the
      // second, so each lane reads its partner's sum from the other half
      const uint64_t b = __builtin_bit_cast(uint64_t, own);
      const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)b, (uint32_t)b, false, false);
      const auto hi =
          __builtin_amdgcn_permlane32_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
      const bool upper = (threadIdx.x & 32) != 0;
      const double partner = __builtin_bit_cast(
          double, (uint64_t)(upper ? lo[0] : lo[1]) | ((uint64_t)(upper ? hi[0] : hi[1]) << 32));
      if (!upper) s_part[wave * 32 + m.kp] = own + partner;
      return upper ? partner : 0.0;
    } else {
      s_part[wave * lay.npair + m.kp] = own;
      return 0.0;
    }
  } else {
    float dt[C::S];
    stage_dt<C>(st, dt);
    if (m.act) s_part[m.blk * lay.npair + m.kp] = item_angle_sum<C::S>(st.th, dt);
    return 0.0;
  }
}

// [R]: rotation items and x items into LDS (consumes the staged registers).
template <class C, bool kWithC, bool kAccumSeg>
__device__ __forceinline__ void step_rotate(const PrefillArgs& a, const PrefillLayout& lay,
                                            const Ctx& s, const Map& m, int c, Stage<C>& st,
                                            const float* sc, const Tiles& t, double inw,
                                            unsigned char* smem) {
  const float* s_w = sc + 3 * kLMax;
  if (m.xact) write_x_item<C>(m.jp, m.xblk, st.x, t.X);
  float dt[C::S];
  stage_dt<C>(st, dt);
  if (m.act)
    rotate_item<C, kWithC, kAccumSeg>(
        lay.npair, lay.nblk, m.kp, m.blk, st.th, dt, st.b, st.c, s_w, t.B, t.C, t.W,
        reinterpret_cast<const double*>(smem + lay.off_part), inw,
        reinterpret_cast<float2*>(smem + lay.off_crot), reinterpret_cast<double*>(smem + lay.off_sang));
}

// ---- chain helpers ---------------------------------------------------------
// This wave's state tiles to / from a state in the workspace (stored tile by
// tile as the waves hold them, prefill_state_index), one 16-byte vector per
// lane and tile, with device-coherent (sc1) buffer stores and loads: the
// other side of the exchange runs on another CU, possibly another XCD.
constexpr int kSc1 = 16;  // cache-policy operand of the buffer intrinsics: sc1
template <class C>
__device__ __forceinline__ void store_state_tiles(const PrefillArgs& a, const WaveRoles& wr,
                                                  const f32x4 (&v)[kMaxStTiles], float* dst) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntiles = (a.N / 16) * C::NPT;
  const rsrc r = make_rsrc(dst, (uint32_t)(a.N * C::P * 4));
#pragma unroll
  for (int q = 0; q < kMaxStTiles; ++q) {
    const int i = state_tile(wr, wave, q, ntiles);
    if (i >= 0)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[q]), r,
                                             (i * 64 + lane) * 16, 0, kSc1);
  }
}
template <class C>
__device__ __forceinline__ void load_state_tiles(const PrefillArgs& a, const WaveRoles& wr,
                                                 const float* src, f32x4 (&v)[kMaxStTiles]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntiles = (a.N / 16) * C::NPT;
  const rsrc r = make_rsrc(src, (uint32_t)(a.N * C::P * 4));
#pragma unroll
  for (int q = 0; q < kMaxStTiles; ++q) {
    v[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int i = state_tile(wr, wave, q, ntiles);
    if (i >= 0)
      v[q] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (i * 64 + lane) * 16, 0, kSc1));
  }
}

// Publish this segment's status word (1 aggregate, 2 exit state) once every
// thread's stores have completed: no writeback fence is needed, since the
// stores and the readers' loads are device-coherent.
__device__ __forceinline__ void publish_status(const PrefillArgs& a, int ticket, int st) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(a.status + ticket, st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until the status words of tickets first - k * stride (k < n) are 1
// and, if last_idx >= 0, the status word of ticket last_idx is 2: one lane
// per word, each wait bounded.  Returns whether every wait succeeded (false:
// a wait timed out and the error word is 1); the answer reaches the
// workgroup through the LDS word s_word.
__device__ __forceinline__ bool wait_statuses(const PrefillArgs& a, int first, int stride, int n,
                                              int last_idx, int* s_word) {
  const int tid = threadIdx.x;
  if (tid == 0) *s_word = 1;
  __syncthreads();
  const int idx = tid < n ? first - tid * stride : (tid == n ? last_idx : -1);
  if (idx >= 0) {
    const int want = tid < n ? 1 : 2;
    int spins = 0;
    while (__hip_atomic_load(a.status + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != want) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_word = 0;
        break;
      }
    }
  }
  __syncthreads();
  return *s_word != 0;
}

// ent += D R v: the accumulated map applied to a state v (an exit state, or
// the continuation's entry), per state tile.
template <class C>
__device__ __forceinline__ void apply_map(const PrefillArgs& a, const WaveRoles& wr,
                                          const float2 (&accr)[kMaxStTiles][2], float accD,
                                          const f32x4 (&v)[kMaxStTiles],
                                          f32x4 (&ent)[kMaxStTiles]) {
#pragma unroll
  for (int q = 0; q < kMaxStTiles; ++q) {
    const float2 r0 = accr[q][0], r1 = accr[q][1];
    const float v0 = accD * v[q][0], v1 = accD * v[q][1];
    const float v2 = accD * v[q][2], v3 = accD * v[q][3];
    ent[q][0] += r0.x * v0 - r0.y * v1;
    ent[q][1] += r0.y * v0 + r0.x * v1;
    ent[q][2] += r1.x * v2 - r1.y * v3;
    ent[q][3] += r1.y * v2 + r1.x * v3;
  }
}

// A predecessor's aggregate as this wave holds it: E per state tile, the
// rotation of each tile's two pairs (lane rows 4g .. 4g+3), the decay.
struct Agg {
  f32x4 v[kMaxStTiles];
  float2 r[kMaxStTiles][2];
  float d;
};

// Request a slot's aggregate (E at slot, rotation and decay at slot + 2NP).
template <class C>
__device__ __forceinline__ void load_agg(const PrefillArgs& a, const WaveRoles& wr,
                                         const float* slot, Agg& g_) {
  load_state_tiles<C>(a, wr, slot, g_.v);
  const float* rd = slot + 2 * (size_t)a.N * C::P;
  const rsrc r = make_rsrc(rd, (uint32_t)(a.N * 4 + 4));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int ntn = a.N / 16, ntiles = ntn * C::NPT;
#pragma unroll
  for (int q = 0; q < kMaxStTiles; ++q) {
    g_.r[q][0] = g_.r[q][1] = make_float2(1.f, 0.f);
    const int i = state_tile(wr, wave, q, ntiles);
    if (i >= 0) {
      // (cos, sin) of pairs kq and kq + 1: one 16-byte vector
      const int kq = (i % ntn) * 8 + 2 * g;
      const f32x4 c = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, kq * 8, 0, kSc1));
      g_.r[q][0] = make_float2(c[0], c[1]);
      g_.r[q][1] = make_float2(c[2], c[3]);
    }
  }
  g_.d = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, a.N * 4, 0, kSc1));
}

// Compose a predecessor's aggregate into the accumulated map: the offset
// gains D R E, then the rotation and decay take the predecessor's.
template <class C>
__device__ __forceinline__ void compose_map(const PrefillArgs& a, const WaveRoles& wr,
                                            const Agg& g_, float2 (&accr)[kMaxStTiles][2],
                                            float& accD, f32x4 (&ent)[kMaxStTiles]) {
  apply_map<C>(a, wr, accr, accD, g_.v, ent);
#pragma unroll
  for (int q = 0; q < kMaxStTiles; ++q)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float2 r = accr[q][k], c = g_.r[q][k];
      accr[q][k] = make_float2(r.x * c.x - r.y * c.y, r.y * c.x + r.x * c.y);
    }
  accD *= g_.d;
}

// Phase 2 of a segment (its chain step), shared by the prefill kernels.
// On entry stt holds this segment's exit state for a zero entry state (its
// local pass), s_srot (LDS, visible to the workgroup) the segment's total
// rotation per pair and segD its total decay.  Each segment's map from entry
// to exit state is x -> R(Phi) D x + E_local (linear recurrence).  Segments
// form groups of kGroup consecutive segments.  Inside a group a segment
// publishes its map (its aggregate) as soon as its local pass is done; the
// group's last segment publishes its exit state instead.  A segment's entry
// state is its group predecessors' maps, composed newest first, applied to
// the previous group's exit state (or to the sequence's start).  So only the
// groups chain one after another, and every entry is computed by the same
// operations on every call (the result does not depend on timing).
// On return ent holds the segment's entry state; for a group's last segment
// (and the sequence's last) stt holds its exit state, which was published
// (or written to h_final).  s_misc: the workgroup's LDS words.
template <class C>
__device__ __forceinline__ void chain_phase(const PrefillArgs& a, const WaveRoles& wr, int seg,
                                            int bh, int ticket, float segD,
                                            const float2* s_srot, int* s_misc,
                                            f32x4 (&stt)[kMaxStTiles],
                                            f32x4 (&ent)[kMaxStTiles]) {
  constexpr int P = C::P;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int npair = a.N / 2;
  const int ntn = a.N / 16, ntiles = ntn * (P / 16);
  const bool last = seg == a.nSeg - 1;
  const bool group_end = seg % kGroup == kGroup - 1;
  const size_t np = (size_t)a.N * P;
  const size_t slotf = prefill_slot_floats(a.N, P);
  float* mine = a.slots + (size_t)ticket * slotf;
#pragma unroll
  for (int q = 0; q < kMaxStTiles; ++q) ent[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (!last && !group_end) {
    // aggregate: E_local, the segment's rotation per pair, its decay
    store_state_tiles<C>(a, wr, stt, mine);
    for (int kp = tid; kp < npair; kp += kT) {
      __hip_atomic_store(mine + 2 * np + 2 * kp, s_srot[kp].x, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(mine + 2 * np + 2 * kp + 1, s_srot[kp].y, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0)
      __hip_atomic_store(mine + 2 * np + a.N, segD, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    publish_status(a, ticket, 1);
  }
  {
    // the accumulated map: per state tile the rotation of its lane's two
    // pairs, one decay, and the accumulated offset (in ent)
    float2 accr[kMaxStTiles][2];
#pragma unroll
    for (int q = 0; q < kMaxStTiles; ++q) accr[q][0] = accr[q][1] = make_float2(1.f, 0.f);
    float accD = 1.f;
    const int BH = a.nb * a.H;
    const int g0 = seg - seg % kGroup;  // first segment of the group
    const int nprev = seg - g0;           // aggregates to compose
    // every wait at once: the group predecessors' aggregates and the
    // previous group's exit state
    const bool ok = wait_statuses(a, (seg - 1) * BH + bh, BH, nprev,
                                  g0 > 0 ? (g0 - 1) * BH + bh : -1, s_misc + 2);
    if (!ok) {
      // a wait timed out (error word 1): the entry state is unknown, so the
      // segment continues from NaN and every y it writes, every state it
      // publishes and h_final are NaN -- a failed call cannot pass for a
      // correct one
#pragma unroll
      for (int q = 0; q < kMaxStTiles; ++q) {
        const float qn = __builtin_nanf("");
        ent[q] = f32x4{qn, qn, qn, qn};
      }
    } else {
      // newest first, several aggregates' loads in flight at a time (fewer
      // with more state per wave: registers)
      constexpr int NB = C::kAggBatch;
      for (int j0 = seg - 1; j0 >= g0; j0 -= NB) {
        Agg ag[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k)
          if (j0 - k >= g0) load_agg<C>(a, wr, a.slots + (size_t)((j0 - k) * BH + bh) * slotf, ag[k]);
#pragma unroll
        for (int k = 0; k < NB; ++k)
          if (j0 - k >= g0) compose_map<C>(a, wr, ag[k], accr, accD, ent);
      }
      // applied to the previous group's exit state, or the sequence's start
      // (zero, or the continuation's entry state)
      if (g0 > 0 || a.cont) {
        const float* src = g0 > 0 ? a.slots + (size_t)((g0 - 1) * BH + bh) * slotf + np
                                  : a.cont_entry + (size_t)bh * np;
        f32x4 v[kMaxStTiles];
        load_state_tiles<C>(a, wr, src, v);
        apply_map<C>(a, wr, accr, accD, v, ent);
      }
    }
  }
  if (last || group_end) {
    // exit state = R(Phi_seg) (D_seg * entry) + local
#pragma unroll
    for (int q = 0; q < kMaxStTiles; ++q) {
      const int i = state_tile(wr, wave, q, ntiles);
      if (i >= 0) {
        const int nt = i % ntn;
        const int kq = nt * 8 + 2 * g;
        const float2 r0 = s_srot[kq], r1 = s_srot[kq + 1];
        f32x4 e;
        const float v0 = segD * ent[q][0], v1 = segD * ent[q][1];
        const float v2 = segD * ent[q][2], v3 = segD * ent[q][3];
        e[0] = r0.x * v0 - r0.y * v1 + stt[q][0];
        e[1] = r0.y * v0 + r0.x * v1 + stt[q][1];
        e[2] = r1.x * v2 - r1.y * v3 + stt[q][2];
        e[3] = r1.y * v2 + r1.x * v3 + stt[q][3];
        stt[q] = e;
      }
    }
    if (!last) {
      store_state_tiles<C>(a, wr, stt, mine + np);
      publish_status(a, ticket, 2);
    } else if (a.h_final) {
#pragma unroll
      for (int q = 0; q < kMaxStTiles; ++q) {
        const int i = state_tile(wr, wave, q, ntiles);
        if (i >= 0) {
          const int nt = i % ntn, pt = i / ntn;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            a.h_final[(size_t)bh * np + (size_t)(nt * 16 + 4 * g + j) * P + pt * 16 + li] =
                stt[q][j];
        }
      }
    }
  }
}

// The last workgroup to finish zeroes the chain counters, so the next call
// on this workspace starts from zeros without a reset launch.  In two
// halves, so that the count's round trip overlaps work that touches no
// counter: finish_count (thread 0 counts the workgroup done; called once the
// workgroup has published and read every status word it touches: its reads
// returned their values, the waits used them, and its own stores are
// complete, s_waitcnt before the count, so the count needs no fence;
// returns the count before it, meaningful in thread 0 only) and
// finish_reset (the zeroing follows the count's returned value, and the next
// call sees it across the kernel boundary).
__device__ __forceinline__ int finish_count(const PrefillArgs& a) {
  int prev = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_s_waitcnt(0);
    prev = atomicAdd(a.done, 1);
  }
  return prev;
}
__device__ __forceinline__ void finish_reset(const PrefillArgs& a, int prev, int* s_misc) {
  const int tid = threadIdx.x;
  if (tid == 0) s_misc[1] = prev == (int)gridDim.x - 1;
  __syncthreads();
  if (s_misc[1]) {
    for (int i = tid; i < (int)gridDim.x; i += kT) a.status[i] = 0;
    if (tid < a.ncls) a.ticket[kTicketStride * tid] = 0;
    if (tid == 0) *a.done = 0;
  }
}

// One workgroup's segment: local exit state, chain, outputs.  `ticket` is
// known to lie inside the grid.
template <class C>
__device__ __forceinline__ int prefill_segment(const PrefillArgs& a, const PrefillLayout& lay,
                                               int ticket, unsigned char* smem) {
  constexpr int P = C::P;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int BH = a.nb * a.H;
  Ctx s0;
  Ctx& s = s0;
  s.seg = ticket / BH;
  s.bh = ticket % BH;
  s.b = s.bh / a.H;
  s.h = s.bh % a.H;
  s.c0 = s.seg * a.K;
  s.c1 = min(a.nC, s.c0 + a.K);
  s.rowB = (uint32_t)(a.H * C::R * a.N * C::es);
  s.rowTh = (uint32_t)(a.H * (a.N / 2) * 4);
  s.rowDt = (uint32_t)(a.H * 4);
  s.rowX = (uint32_t)(a.H * C::R * P * C::es);
  // a uniform value, taken into a scalar register here so that its load is
  // complete before the chunk loops
  s.Ah = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.A[s.h])));

  Map m;
  m.act = tid < lay.items;
  m.kp = tid % lay.npair;
  m.blk = tid / lay.npair;
  m.xact = tid < lay.xitems;
  m.jp = tid % (P / 2);
  m.xblk = tid / (P / 2);
  m.xwave = __builtin_amdgcn_readfirstlane(wave) * kWave < lay.xitems;
  m.wblk = __builtin_amdgcn_readfirstlane(wave * kWave / lay.npair);

  const Tiles tiles0 = make_tiles<C>(a, lay, smem);
  const Tiles& t = tiles0;
  const WaveRoles wr = prefill_wave_roles(lay.LR, P);
  float* s_scal = reinterpret_cast<float*>(smem + lay.off_scal);
  double* s_sang = reinterpret_cast<double*>(smem + lay.off_sang);
  float2* s_srot = reinterpret_cast<float2*>(smem + lay.off_srot);
  const int npair = lay.npair;
  const int ntn = a.N / 16, ntiles = ntn * (P / 16);

  // zero the K-major tiles past the chunk's rows (never written again): the
  // contraction padding, and the rest of a fixed-length row, which the key
  // blocks of a chunk shorter than 32 rows read past the end of B~ and only
  // mask out (so it must hold finite values)
  if (lay.KM > lay.LR) {
    const int padb = (lay.KM - lay.LR) * C::es;  // bytes per row, a multiple of 16
    const int per = padb / 16;
    for (int i = tid; i < (a.N + P) * per; i += kT) {
      const int row = i / per, col = i % per;
      const Tile& tt = row < a.N ? t.W : t.X;
      const int rr = row < a.N ? row : row - a.N;
      tt.ref<u32x4>((uint32_t)rr, (uint32_t)(lay.LR * C::es + col * 16)) = u32x4{0u, 0u, 0u, 0u};
    }
  }
  for (int i = tid; i < npair; i += kT) s_sang[i] = 0.0;
  // the output pass's score hand-over, if it applies (its counter starts at
  // zero; many barriers pass before the output pass)
  ScoreX hx{reinterpret_cast<uint32_t*>(smem + lay.off_sx),
            reinterpret_cast<int*>(smem + lay.off_sx + kScoreXBytes - 16), 0};
  const bool hand = C::kHand3 && prefill_score_handover(a.L, C::R, a.N, P, C::NC != 0) &&
                    prefill_wave_roles(lay.LR, P).nout == kW / 2;
  if (hand && tid == 0) *hx.flag = 0;

  f32x4 stt[kMaxStTiles];
#pragma unroll
  for (int q = 0; q < kMaxStTiles; ++q) stt[q] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- phase 1: local exit state of the segment --------------------------
  Stage<C> stg;
  issue_loads<C, false>(a, s, m, s.c0, stg);
  const bool scal_wave = __builtin_amdgcn_readfirstlane(tid >> 6) == kScalarWave;
  constexpr int NJ = C::NC != 0 ? 2 : 3;  // N fixed: chunks of at most 64 tokens
  if (scal_wave) {
    float wd[3], wl[3];
    scalar_loads<NJ>(a, s, s.c0, wd, wl, true);
    const int t0c = s.c0 * a.L;
    chunk_scalars(a, t0c, min(a.L, a.T - t0c), s.Ah, wd, wl, s_scal);
  }
  float seg_logdecay = 0.f;
  int buf = 0;
  for (int c = s.c0; c < s.c1; ++c) {
    float* sc = s_scal + buf * (kScalBytes / 4);
    const Ctx s = step_ctx(s0);
    const Tiles t = step_tiles<C>(tiles0, smem);
    const double inw = step_partials<C>(a, lay, s, m, c, stg, sc, smem);
    // the next chunk's dt and lam (the first chunk's again after the last,
    // for phase 3), for the scalar wave, requested once the staged angles
    // are summed: they have the rest of the step to arrive, and are not
    // queued behind the next chunk's staging loads.  Every wave issues these
    // loads (the others over an empty range, which reads zeros without a
    // memory access), so that each wave has the same loads in flight where
    // it waits for its staged registers
    const int nc = c + 1 < s.c1 ? c + 1 : s.c0;
    float wd[3], wl[3];
    scalar_loads<NJ>(a, s, nc, wd, wl, scal_wave);
    __syncthreads();
    step_rotate<C, false, true>(a, lay, s, m, c, stg, sc, t, inw, smem);
    // prefetch the next chunk; the last step prefetches the first chunk
    // again, with C, for phase 3
    if (c + 1 < s.c1)
      issue_loads<C, false>(a, s, m, c + 1, stg);
    else
      issue_loads<C, true>(a, s, m, s.c0, stg);
    __syncthreads();
    const float lc = sc[4 * kLMax];
    seg_logdecay += lc;
    state_update<C>(a, lay, wr, __expf(lc), stt, t.W, t.X, smem);
    // the scalar wave prepares the next chunk's scalars in the other buffer
    if (scal_wave)
      chunk_scalars(a, nc * a.L, min(a.L, a.T - nc * a.L), s.Ah, wd, wl,
                    s_scal + (buf ^ 1) * (kScalBytes / 4));
    buf ^= 1;
  }

  // ---- phase 2: chain (look-back in groups; see chain_phase) ---------------
  __syncthreads();
  for (int kp = tid; kp < npair; kp += kT) {
    float sn, cn;
    sincosf(static_cast<float>(s_sang[kp]), &sn, &cn);
    s_srot[kp] = make_float2(cn, sn);
  }
  const float segD = __expf(seg_logdecay);
  int* s_misc = reinterpret_cast<int*>(smem + lay.off_misc);
  f32x4 ent[kMaxStTiles];
  __syncthreads();  // s_srot
  chain_phase<C>(a, wr, s.seg, s.bh, ticket, segD, s_srot, s_misc, stt, ent);
  // every load of the chain has returned (a load whose value the chain did
  // not need would otherwise leave the compiler a pending write to its
  // register, waited for inside the output pass)
  __builtin_amdgcn_s_waitcnt(0);
  // no counter is touched after the chain: the workgroup counts itself done
  // here, and the count's round trip overlaps the output pass
  const int done_prev = finish_count(a);
  // the output pass's state distribution (see Cfg::kSplit3): the entry
  // state moves to its waves through LDS
  WaveRoles wr3 = wr;
  if constexpr (C::kSplit3) {
    wr3.sw0 = kW / 2;
    wr3.nsw = kW / 2;
    float* s_hand = reinterpret_cast<float*>(smem + lay.off_hand);
#pragma unroll
    for (int q = 0; q < kMaxStTiles; ++q) {
      const int i = state_tile(wr, wave, q, ntiles);
      if (i >= 0) *reinterpret_cast<f32x4*>(s_hand + (i * 64 + lane) * 4) = ent[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kMaxStTiles; ++q) {
      const int i = state_tile(wr3, wave, q, ntiles);
      stt[q] = i >= 0 ? *reinterpret_cast<const f32x4*>(s_hand + (i * 64 + lane) * 4)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  } else {
#pragma unroll
    for (int q = 0; q < kMaxStTiles; ++q) stt[q] = ent[q];
  }
  constexpr int NSW3 = C::kSplit3 ? kW / 2 : kW;
  // Waves kW/2.. share SIMDs with the older waves 0 .. kW/2-1, which issue
  // first, so their rotation step ends later, and the older waves would wait
  // for their load requests at the step's second barrier.  With the score
  // hand-over (no output unit on them) they request the next chunk's inputs
  // after their scores; with sixteen units dealt unevenly (see chunk_output)
  // right after the barrier, before their smaller units.
  const bool late = hand && __builtin_amdgcn_readfirstlane(wave) >= kW / 2;
  const bool late16 = C::kDeal16 && wr.nout == 2 * kW && wr.npg == 1 &&
                      __builtin_amdgcn_readfirstlane(wave) >= kW / 2;

  // ---- phase 3: outputs from the true entry state -------------------------
  for (int c = s.c0; c < s.c1; ++c) {
    float* sc = s_scal + buf * (kScalBytes / 4);
    const bool more = c + 1 < s.c1;
    const Ctx s = step_ctx(s0);
    const Tiles t = step_tiles<C>(tiles0, smem);
    const double inw = step_partials<C>(a, lay, s, m, c, stg, sc, smem);
    float wd[3], wl[3];
    scalar_loads<NJ>(a, s, more ? c + 1 : c, wd, wl, more && scal_wave);
    __syncthreads();
    step_rotate<C, true, false>(a, lay, s, m, c, stg, sc, t, inw, smem);
    state_to_lds<C>(a, wr3, stt, t.G);
    if (more && !late && !late16) issue_loads<C, true>(a, s, m, c + 1, stg);
    __syncthreads();
    if (more && late16) issue_loads<C, true>(a, s, m, c + 1, stg);
    hx.target = hand ? 4 * (c - s.c0 + 1) : 0;
    chunk_output<C>(a, lay, wr, s, chunk_res<C>(a, s, c), sc, t.C, t.B, t.X, t.G, hx);
    if (more) {
      if (late) issue_loads<C, true>(a, s, m, c + 1, stg);
      state_update<C, NSW3>(a, lay, wr3, __expf(sc[4 * kLMax]), stt, t.W, t.X, smem);
      if (scal_wave)
        chunk_scalars(a, (c + 1) * a.L, min(a.L, a.T - (c + 1) * a.L), s.Ah, wd, wl,
                      s_scal + (buf ^ 1) * (kScalBytes / 4));
    }
    buf ^= 1;
  }
  return done_prev;
}

// The workgroup's ticket (its segment), or -1.  Only the holder of a ticket
// writes its status word, and the previous call's last workgroup zeroed it,
// so the word is zero here on a clean workspace.  A ticket outside the grid
// (the ticket word was not zero at entry) or a nonzero status word of its
// own means dirty counters: the caller reports it (bad_ticket) and touches
// nothing else.  s_misc: two ints of LDS.
// The status word of ticket blockIdx.x is read together with the ticket,
// before knowing it: workgroups mostly draw the ticket of their own index,
// and then the check costs no second round trip to the device-coherent
// level (reading it early is harmless: only the ticket's holder writes it).
__device__ __forceinline__ int take_ticket(const PrefillArgs& a, int* s_misc) {
  if (threadIdx.x == 0) {
    const int guess = (int)blockIdx.x;
    const int st_guess = __hip_atomic_load(a.status + guess, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the class's counter (see kTicketStride): its workgroups, in the order
    // they come, take the class's tickets in increasing order
    const int cls = guess & (a.ncls - 1);
    int t = cls + a.ncls * atomicAdd(a.ticket + kTicketStride * cls, 1);
    if (t >= 0 && t < (int)gridDim.x) {
      const int st = t == guess ? st_guess
                                : __hip_atomic_load(a.status + t, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
      if (st != 0) t = -1;
    }
    s_misc[0] = t;
  }
  __syncthreads();
  return s_misc[0];
}
__device__ __forceinline__ void bad_ticket(const PrefillArgs& a) {
  if (threadIdx.x == 0) __hip_atomic_store(a.err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class C>
__global__ void __launch_bounds__(kT) prefill_kernel(PrefillArgs a_in) {
  extern __shared__ __align__(16) unsigned char smem[];
  // with N fixed at compile time every contraction loop over N unrolls and
  // the pair / block index arithmetic folds
  PrefillArgs a = a_in;
  if constexpr (C::NC != 0) a.N = C::NC;
  const PrefillLayout lay = prefill_layout(a.L, C::R, a.N, C::P, C::es, C::NC != 0);
  int* s_misc = reinterpret_cast<int*>(smem + lay.off_misc);
  // (the range test stays at the call: the segment code is compiled knowing
  // the ticket lies in the grid)
  const int ticket = take_ticket(a, s_misc);
  int done_prev;
  if (ticket >= 0 && ticket < (int)gridDim.x) {
    done_prev = prefill_segment<C>(a, lay, ticket, smem);
  } else {
    bad_ticket(a);
    done_prev = finish_count(a);
  }
  finish_reset(a, done_prev, s_misc);
}

template <class C>
hipError_t launch_cfg(const PrefillArgs& a, hipStream_t stream) {
  const PrefillLayout lay = prefill_layout(a.L, C::R, a.N, C::P, C::es, C::NC != 0);
  hipError_t e = lds_limit(reinterpret_cast<const void*>(&prefill_kernel<C>), lay.total);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_kernel<C>), dim3(a.nb * a.H * a.nSeg), dim3(kT), lay.total, stream,
                     a);
  return hipGetLastError();
}

}  // namespace pf

// bfloat16, R = 1, N = 128 fixed: compiled on its own
// (prefill_bf16_r1_n128.hip) so that it can take other scheduling options.
hipError_t launch_prefill_bf16_r1_n128(const PrefillArgs& a, hipStream_t stream);

namespace pf {

// bfloat16 (the fast path) has instantiations with N fixed for the common
// state sizes and chunks of at most 64 tokens (every tile geometry a
// compile-time constant); float32 and other shapes take N at run time.
template <typename T, int R, int P>
hipError_t launch_trp(const PrefillArgs& a, hipStream_t stream) {
  if constexpr (sizeof(T) == 2) {
    const PrefillLayout fl = prefill_layout(a.L, R, a.N, P, 2, true);
    if (prefill_fixed_shape(a.L, a.N, 2) && fl.total <= kLdsLimit &&
        fl.items <= kPrefillThreads && fl.xitems <= kPrefillThreads)
      switch (a.N) {
        case 64: return launch_cfg<Cfg<T, R, P, 64>>(a, stream);
        case 128:
          if constexpr (R == 1) return launch_prefill_bf16_r1_n128(a, stream);
          else return launch_cfg<Cfg<T, R, P, 128>>(a, stream);
        default: break;
      }
  }
  return launch_cfg<Cfg<T, R, P, 0>>(a, stream);
}

template <typename T, int R>
hipError_t launch_tr(const PrefillArgs& a, hipStream_t stream) {
  switch (a.P) {
    case 16: return launch_trp<T, R, 16>(a, stream);
    case 32: return launch_trp<T, R, 32>(a, stream);
    case 64: return launch_trp<T, R, 64>(a, stream);
    case 128: return launch_trp<T, R, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  switch (a.R) {
    case 1: return launch_tr<T, 1>(a, stream);
    case 2: return launch_tr<T, 2>(a, stream);
    case 4: return launch_tr<T, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pf
}  // namespace m3
