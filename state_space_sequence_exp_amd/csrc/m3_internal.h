// m3_internal.h -- host-side interface between the C ABI (m3ssm_api.hip) and
// the kernel launchers.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "m3ssm.h"

namespace m3 {

#ifndef M3_PREFILL_THREADS
#define M3_PREFILL_THREADS 512
#endif
constexpr int kPrefillThreads = M3_PREFILL_THREADS;  // threads per prefill workgroup (one per CU)
constexpr int kLMax = 128;                // largest chunk (tokens)
constexpr int kLRMax = 256;               // largest chunk * R (rows of a chunk tile)
constexpr size_t kLdsLimit = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int kMaxStTiles = 8192 / 256 / (kPrefillThreads / 64);  // 16x16 state tiles per wave (N * P <= 8192)

// Raise kernel `fn`'s dynamic LDS limit to at least `bytes` on the current
// device.  The limit is an attribute of the function on a device, not of a
// launch, so the runtime call is made only the first time a (function,
// device) pair needs a larger limit; later launches take a lock-guarded look
// at a small table.
hipError_t lds_limit(const void* fn, size_t bytes);

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
  const float* h0;      // [B*H][N][P] state before the first token, or null (zero)
  const void* x_prev;   // [B*H][R][P] input of the token before the first, or null (zero)
  const void* B_prev;   // [B*H][R][N] its B (null exactly when x_prev is)
  int cont;             // 1: the entry kernel staged each sequence's entry state in cont_entry
  void* y;
  float* h_final;
  // workspace carve
  float* slots;       // [grid] per segment (ticket): aggregate E [N][P], exit state [N][P],
                      //        rotation (cos, sin) per pair [N/2][2], decay, 3 unused
  float* cont_entry;  // [B*H][N][P] entry state of each sequence's first segment (cont)
  int* status;        // [grid] per ticket: 0 nothing, 1 aggregate, 2 exit state published
  int* ticket;        // ticket counters: class c's at ticket[kTicketStride c] (work order)
  int* err;           // [1]   1: a wait for a predecessor timed out; 2: counters not zero at entry
  int* done;          // [1]   finished workgroups; the last one zeroes status, tickets, done
  int ncls;           // ticket classes in use (a power of two dividing nb * H, at most 8)
};

// The prefill workspace's chain counters (int32 words).  Workgroups take
// their tickets from one counter per class: workgroup b is in class b %
// ncls and draws ticket c + ncls k from class c's counter, so a segment's
// predecessors in its sequence (tickets t - j nb H, the same class when
// ncls divides nb H) are drawn from its own counter, before its own.  Each
// counter has a 128-byte line of its own, so the workgroups of a launch do
// not all queue on one address.  Class 0's counter is word 0, the error word
// 1 and the finished-workgroup count 2; class c's counter is word
// kTicketStride c; the status words start at kStatusWord; the segments'
// slots start at kSlotsMinBytes or past the status words.
constexpr int kTicketClasses = 8;
constexpr int kTicketStride = 32;
constexpr int kStatusWord = kTicketClasses * kTicketStride;
constexpr size_t kSlotsMinBytes = 8192;

// Ticket classes for nb * H sequences: the largest power of two up to
// kTicketClasses that divides it.
__host__ __device__ constexpr int prefill_ticket_classes(long long units) {
  return units % 8 == 0 ? 8 : (units % 4 == 0 ? 4 : (units % 2 == 0 ? 2 : 1));
}

// Floats of one segment's slot in the prefill workspace.
__host__ __device__ constexpr size_t prefill_slot_floats(int N, int P) {
  return 2 * (size_t)N * P + (size_t)N + 4;
}

// Position of state element (n, p) in the workspace's states (the slots and
// the entry states), which are stored the way the prefill kernel's waves
// hold them: 16 x 16 tile i = (p / 16) (N / 16) + n / 16, then lane
// 16 ((n % 16) / 4) + p % 16, then n % 4, so a lane's four values are one
// 16-byte vector.
__host__ __device__ inline size_t prefill_state_index(int N, int n, int p) {
  const int i = (p / 16) * (N / 16) + n / 16;
  const int lane = 16 * ((n % 16) / 4) + p % 16;
  return ((size_t)i * 64 + lane) * 4 + n % 4;
}

struct DecodeArgs {
  int S, H, P, N, R;
  const float* h_in;
  float* h_out;
  const void *x_t, *x_prev, *B_t, *B_prev, *C_t;
  const float *dt, *A, *lam, *theta;
  void* y;
};
// The decode step with its rank-2R update on the matrix cores (decode.hip):
// the shapes it takes, and its launch (hipErrorInvalidValue for others).
bool decode_mfma_shape(int R, int N, int P);
hipError_t launch_decode_mfma(const DecodeArgs& a, m3_dtype dtype, hipStream_t stream);


// Gradients of the recurrence (backward.hip).
struct BackwardArgs {
  int nb, T, H, P, N, R;
  const void *x, *B, *C, *dy;                       // storage type of the call
  const float *dt, *A, *lam, *theta, *dh_final;     // dh_final may be null
  float *dx, *ddt, *dA, *dlam, *dtheta, *dB, *dC;   // gradients, float
  // workspace: the states (every token's h_t and G_t, or with segments of S
  // tokens the segment-entry h and segment-exit dU checkpoints) and the
  // per-token dA terms
  float *hs, *gs, *dAc;
  int S;  // segment length of the checkpointed path (0: states per token)
  // per segment: its decay prod_t alpha_t and, per row pair, its rotation
  // angle sum_t dt_t theta_t (checkpointed path)
  float *dseg, *psi;
  // chunked path (L > 0, chunks of L tokens, backward_chunk.hip): hs holds
  // the entry states of chunks 0 .. nC, gs the exit adjoints of chunks
  // 0 .. nC - 1, dseg per chunk the cosines and sines of its total rotation
  // and its decay (65 floats), dAc four per-token partial arrays
  int L;
};

// Shapes the chunked backward takes: N = P = 64 (64-column tiles), R of 1, 2
// or 4 (chunks of 64 / R tokens).
__host__ __device__ inline bool bw_chunked_shape(int R, int N, int P) {
  return N == 64 && P == 64 && (R == 1 || R == 2 || R == 4);
}
hipError_t launch_backward_chunked(const BackwardArgs& a, m3_dtype dtype, hipStream_t stream);

// Segment path of the backward: one workgroup of N P / (2 W) threads per
// (sequence, head, segment of S tokens); thread (kp, q) holds rows 2 kp,
// 2 kp + 1 and columns W q .. W q + W - 1 of the state (W = 4).  Tokens are
// recomputed in blocks of kBwSub.
constexpr int kBwSub = 8;
constexpr int kBwMaxThreads = 512;  // at W = 4

// LDS of one segment workgroup (byte offsets, 16-aligned): the segment's
// inputs for tokens t0 - 1 .. t0 + S (S + 2 slots) as stored; for nbuf
// blocks (with two, alternate blocks use alternate halves and one barrier
// per block suffices), the per-wave dx partials, per-row-pair scalar
// partials and the dB, dC and dtheta rows; a 16-byte slot per lane that the
// lanes with nothing to store write instead (so the stores need no branch);
// each thread's block-entry states.
struct BwSegLayout {
  int nslot;
  uint32_t wB, wX;  // 32-bit words per token-head row of B (and C), of x (and dy)
  size_t oB, oC, oX, oDY, oTh, oDt, oLam, oDx, oSc, odB, odC, odTh, oNull, oHs, total;
};

__host__ __device__ inline BwSegLayout bw_seg_layout(int S, int R, int N, int P, int es,
                                                     int W = 4, int nbuf = 1) {
  BwSegLayout l;
  const int nt = N * P / (2 * W), nw = (nt + 63) / 64;
  l.nslot = S + 2;
  l.wB = (uint32_t)(R * N * es / 4);
  l.wX = (uint32_t)(R * P * es / 4);
  size_t o = 0;
  auto take = [&o](size_t bytes) {
    const size_t at = o;
    o = (o + bytes + 15) / 16 * 16;
    return at;
  };
  l.oB = take((size_t)l.nslot * l.wB * 4);
  l.oC = take((size_t)l.nslot * l.wB * 4);
  l.oX = take((size_t)l.nslot * l.wX * 4);
  l.oDY = take((size_t)l.nslot * l.wX * 4);
  l.oTh = take((size_t)l.nslot * (N / 2) * 4);
  l.oDt = take((size_t)l.nslot * 4);
  l.oLam = take((size_t)l.nslot * 4);
  l.oDx = take(nbuf * (size_t)nw * kBwSub * R * P * 4);
  l.oSc = take(nbuf * (size_t)(N / 2) * kBwSub * 16);
  l.odB = take(nbuf * (size_t)kBwSub * R * N * 4);
  l.odC = take(nbuf * (size_t)kBwSub * R * N * 4);
  l.odTh = take(nbuf * (size_t)kBwSub * (N / 2) * 4);
  l.oNull = take(64 * 16);
  l.oHs = take((size_t)(S / kBwSub) * 2 * W * nt * 4);
  l.total = o;
  return l;
}

// Segment length of the backward's checkpointed path for a shape (32, else
// 16 or 8 to fit the LDS), or 0 when the shape takes the per-token states
// (N P > 8 kBwMaxThreads).
__host__ __device__ inline int bw_segment_len(int R, int N, int P, int es) {
  if (N * P > 8 * kBwMaxThreads || P < 16) return 0;
  for (int S = 32; S >= kBwSub; S /= 2)
    if (bw_seg_layout(S, R, N, P, es).total <= kLdsLimit) return S;
  return 0;
}

// Blocks' worth of partial-sum rows the gradient pass keeps at segment
// length S: 2 where they fit the LDS, else 1.
__host__ __device__ inline int bw_seg_buffers(int S, int R, int N, int P, int es) {
  return bw_seg_layout(S, R, N, P, es, 4, 2).total <= kLdsLimit ? 2 : 1;
}



// Block-side passes (BCNorm + bias, MIMO projections).
struct BlockArgs {
  size_t rows;  // batch * seqlen * H token-head rows
  int H, P, N, R;
  float eps;
  const void *x, *B, *C;                                     // pre-pass inputs
  const float *norm_B, *norm_C, *bias_B, *bias_C, *up;      // pre-pass weights
  void *x_out, *B_out, *C_out;                               // pre-pass outputs
  const void* y;                                             // post-pass input
  const float* down;                                         // post-pass weights
  void* y_out;                                               // post-pass output
};

__host__ __device__ inline uint32_t align_up_u32(uint32_t v, uint32_t a) {
  return (v + a - 1) / a * a;
}

// Tokens per rotation item: one thread rotates one pair of B (and C) rows
// over this many consecutive tokens (and all R ranks of each token).
__host__ __device__ constexpr int prefill_item_tokens(int esize, int R, int N = 0, int P = 0) {
  // tokens per item at 1024 threads, times 1024 / threads; the instantiation
  // with N = 64 (and P <= 64) fixed, R = 1 and bfloat16 takes chunks of at
  // most 64 tokens and half that many (at 512 threads 32 pairs x 16 blocks of
  // 4 tokens give every thread a rotation item and an x item)
  return (esize == 2 ? (R == 1 ? 4 : 2) : (R == 4 ? 1 : 4 / R)) * (1024 / kPrefillThreads) /
         ((esize == 2 && R == 1 && N == 64 && P != 0 && P <= 64 && kPrefillThreads < 1024) ? 2
                                                                                         : 1);
}

// Per-token scalars of one chunk, one of two alternating buffers:
// cs, gamma, gamma + omega and the state weight w (kLMax floats each), then
// the chunk's log-decay.
constexpr uint32_t kScalBytes = (4 * kLMax + 4) * 4;

// LDS layout of the prefill workgroup, identical on host and device.  The
// five chunk tiles are stored without padding; their 16-byte columns are
// XOR-swizzled by row (see the kernel) so MFMA fragment reads do not
// collide in the LDS banks.
struct PrefillLayout {
  int LR;      // rows of a chunk tile (tokens * R)
  int LRp;     // LR rounded up to the MFMA contraction length
  int S;       // tokens per rotation item
  int npair;   // N / 2
  int nblk;    // token blocks per chunk (L / S)
  int items;   // rotation items (npair * nblk)
  int xitems;  // x items ((P / 2) * nblk)
  uint32_t off_scal;   // 2 x kScalBytes
  uint32_t off_part;   // per-item (or per-wave) angle sums, doubles
  uint32_t off_crot;   // npair float2: (cos, sin) of the chunk's total angle
  uint32_t off_srot;   // npair float2: (cos, sin) of the segment's total angle
  uint32_t off_sang;   // npair doubles: segment angle sums
  uint32_t off_misc;   // 16 bytes: the workgroup's ticket
  uint32_t off_Cr;     // [LR][N]   C~ (rotated C)
  uint32_t off_Br;     // [LR][N]   B~ (rotated B)
  int KM;      // row length (elements) of the two contraction-major tiles
  uint32_t off_BwT;    // [N][KM]   B~ weighted by each token's state weight, transposed
  uint32_t off_XT;     // [P][KM]   x transposed
  uint32_t off_GT;     // [P][N]    chunk entry state, transposed
  uint32_t off_hand;   // N P floats: the entry state handed between wave layouts (N = 64
                       // fixed, P <= 64, R = 1), else empty
  uint32_t off_sx;     // kScoreXBytes: scores handed between waves in the output pass
                       // (see prefill_score_handover), else empty
  uint32_t total;
};

// With N = 128 fixed, R = 1, P <= 64 and chunks of 64 tokens the output pass
// has one unit per query block (all of its p-tiles), on four of the eight
// waves.  Four of the others then compute the masked scores of the two last
// query blocks against the first key pair, one 16 x 16 block each, and hand
// them over through LDS: 4 blocks of 64 lanes x 4 bfloat16, then a counter.
constexpr uint32_t kScoreXBytes = 4 * 64 * 8 + 16;
__host__ __device__ constexpr bool prefill_score_handover(int L, int R, int N, int P, bool fixed) {
  return fixed && N == 128 && R == 1 && L == 64 && P <= 64 && kPrefillThreads == 512;
}

// Whether the kernel instantiated with N fixed at compile time takes the
// shape: bfloat16, N of 64 or 128 and a chunk of at most 64 tokens, whose
// contraction-major tiles then have a fixed row of 64 R elements, so every
// tile's geometry is a compile-time constant.
__host__ __device__ constexpr bool prefill_fixed_shape(int L, int N, int esize) {
  return esize == 2 && (N == 64 || N == 128) && L <= 64;
}

__host__ __device__ inline PrefillLayout prefill_layout(int L, int R, int N, int P, int esize,
                                                        bool fixed = false) {
  PrefillLayout c;
  c.LR = L * R;
  c.LRp = esize == 2 ? (c.LR + 31) / 32 * 32 : c.LR;
  c.KM = fixed ? 64 * R : c.LRp;
  c.S = fixed ? prefill_item_tokens(esize, R, N, P) : prefill_item_tokens(esize, R);
  c.npair = N / 2;
  c.nblk = L / c.S;
  c.items = c.npair * c.nblk;
  c.xitems = (P / 2) * c.nblk;
  uint32_t o = 0;
  c.off_scal = o; o += 2 * kScalBytes;
  // (with N fixed, at least one double per pair and wave: the waves' totals)
  const int nsum = fixed && c.npair * (kPrefillThreads / 64) > c.items ? c.npair * (kPrefillThreads / 64)
                                                                        : c.items;
  c.off_part = o; o += (uint32_t)nsum * 8;
  c.off_crot = o; o += (uint32_t)c.npair * 8;
  c.off_srot = o; o += (uint32_t)c.npair * 8;
  c.off_sang = o; o += (uint32_t)c.npair * 8;
  c.off_misc = o; o += 16;
  o = align_up_u32(o, 16);
  c.off_Cr = o; o += (uint32_t)c.LR * N * esize;
  c.off_Br = o; o += (uint32_t)c.LR * N * esize;
  c.off_BwT = o; o += (uint32_t)N * c.KM * esize;
  c.off_XT = o; o += (uint32_t)P * c.KM * esize;
  c.off_GT = o; o += (uint32_t)P * N * esize;
  c.off_hand = o;
  if (fixed && N == 64 && P <= 64 && R == 1) o += (uint32_t)N * P * 4;
  c.off_sx = o;
  if (prefill_score_handover(L, R, N, P, fixed)) o += kScoreXBytes;
  c.total = o;
  return c;
}

// Roles of the waves in a chunk's MFMA phase.  The outputs are split into
// units of one 16-row query block and a group of at most four p-tiles; with
// few query blocks a unit covers as many p-tiles as it can (each query
// block's scores are then computed once), otherwise two, and units are dealt
// to the waves from wave 0.  The state tiles are spread over all waves
// (tile i on wave i % waves).
struct WaveRoles {
  int ppg;   // p-tiles per unit
  int npg;   // units per query block
  int nout;  // output units
  int sw0;   // first wave holding state tiles
  int nsw;   // waves holding state tiles
};
__host__ __device__ inline WaveRoles prefill_wave_roles(int LR, int P) {
  constexpr int kW = kPrefillThreads / 64;
  const int nqb = LR / 16, npt = P / 16;
  WaveRoles w;
  // units of up to four p-tiles (each query block's scores computed once)
  // where the query blocks are few, or many enough that the zigzag dealing
  // still gives every wave two units of balanced cost; two p-tiles between
  // (one unit of four per wave would leave the causal cost unbalanced)
  const int cap = (nqb * 2 <= kW || (kW <= 4 && nqb <= kW) || nqb >= 2 * kW) ? 4 : 2;
  w.ppg = npt < cap ? npt : cap;
  w.npg = npt / w.ppg;
  w.nout = nqb * w.npg;
  w.sw0 = 0;
  w.nsw = kW - w.sw0;
  return w;
}

// Shapes the prefill kernel handles beyond the LDS limit: at most
// kMaxStTiles state tiles per state wave, at most one rotation item and one x
// item per thread, and byte offsets within one chunk that fit 30 bits.
__host__ __device__ inline bool prefill_shape_fits(int L, int R, int N, int P, int H, int esize) {
  const PrefillLayout lay = prefill_layout(L, R, N, P, esize);
  const WaveRoles w = prefill_wave_roles(lay.LR, P);
  const long long row = (long long)H * R * (N > P ? N : P) * esize;
  return (N / 16) * (P / 16) <= 32 && (N / 16) * (P / 16) <= kMaxStTiles * w.nsw &&
         lay.items <= kPrefillThreads && lay.xitems <= kPrefillThreads &&
         (long long)L * row < (1ll << 30);
}

hipError_t launch_prefill(const PrefillArgs& a, m3_dtype dtype, hipStream_t stream);
hipError_t launch_block_prepass(const BlockArgs& a, m3_dtype dtype, hipStream_t stream);
hipError_t launch_backward(const BackwardArgs& a, m3_dtype dtype, hipStream_t stream);
hipError_t launch_block_postpass(const BlockArgs& a, m3_dtype dtype, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, m3_dtype dtype, hipStream_t stream);

// Per-type (and, for bfloat16, per-rank) prefill launchers, one translation
// unit each.
hipError_t launch_prefill_bf16_r1(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_bf16_r2(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_bf16_r4(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);
// The token-lane kernel (prefill_tok.h) for the shapes it takes (bfloat16,
// rank 1, 64-token chunks, N = P = 64): *taken says whether it took the
// shape (else nothing was launched).
hipError_t launch_prefill_tok(const PrefillArgs& a, hipStream_t stream, bool* taken);

// Largest N the decode kernel handles for a given P.
int decode_max_n(int P);

// Chunks per segment (one prefill workgroup walks one segment).
int prefill_segment_chunks(int nb, int H, int nC);

}  // namespace m3
