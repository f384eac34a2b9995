// prefill_tok.h -- the token-lane prefill kernel: the fused chunked prefill of
// prefill_impl.h re-laid out for 64-token chunks of bfloat16 inputs with state
// size and head dimension 64 and rank 1 (the shape it runs faster than that
// kernel; the others keep it).  Same segments, same chain (chain_phase),
// same workspace; what changes is how a chunk step maps onto the waves and
// how its inputs reach the LDS.
//
// Lane = token.  A chunk has 64 tokens, a wave 64 lanes: lane u of every wave
// works on token u, and wave w owns a group of N/16 rotation pairs of every
// token.  So:
//  * the per-token scalars -- the log-decay prefix cs_u (a wave scan of
//    dt_u A), gamma_u = lam_u dt_u, omega_u = (1 - lam_{u+1}) dt_{u+1} and the
//    state weight exp(cs_e - cs_u)(gamma_u + omega_u) -- are computed by every
//    wave in registers (the exponential-trapezoidal weights of Proposition 1,
//    Mamba-3 paper summary);
//  * the chunk-local cumulative angle of each pair is a wave scan over the
//    lanes of dt_u theta_u[k] in revolutions (the data-dependent RoPE of
//    Proposition 3), reduced modulo one revolution between the in-row and the
//    cross-row steps, so no other wave and no barrier is involved;
//  * each lane rotates its pairs of B (and C) -- two bf16 dot products per
//    pair, with the cosine and sine rounded to bf16 -- and writes whole
//    16-byte pieces of row-major [token][N] tiles: B~ and C~ for the scores,
//    B~ weighted by the state weight for the chunk state.
// The contractions over tokens (the chunk state S = sum_u w_u B~_u x_u^T and
// the output's masked scores times x) need their operands K(token)-major;
// gfx950's LDS transpose read (ds_read_b64_tr_b16) delivers them from the
// row-major tiles, so no tile is ever written transposed.  Outputs are
// computed transposed (p x queries), so each lane holds four consecutive p
// of one token and stores them as one 8-byte vector.
//
// Staging.  A chunk's inputs reach the LDS through direct global-to-LDS
// loads (buffer_load_dwordx4 ... lds): each lane moves 16 bytes to its own
// 16-byte slot of a 1 KB block, and the lane-to-address map is chosen so that
// eight consecutive lanes read one whole 128-byte token row -- coalesced --
// while the block lands already XOR-swizzled, as the row-major tiles are laid
// out.  Rows past the sequence's end are outside the buffer range and land
// as zeros.  So the loads take no registers, and the token-major reads of the
// rotation step come from the LDS.  Each chunk has a buffer of a ring of
// three (B, rotated in place into B~; C, rotated in place into C~; the
// weighted B~; x; theta; dt and lam; the per-token scalars; the chunk's
// rotation; the entry state).  A step is [rotate chunk c: read and write
// buffer c] -- barrier -- [MFMA: read buffer c; then issue the loads of chunk
// c + 2], so one barrier per chunk suffices, waves that finish their MFMA
// work go on to rotate the next chunk while others still multiply, and the
// loads have the next step to arrive.
#pragma once

#include "prefill_impl.h"

namespace m3 {
namespace pt {

using pf::make_rsrc;
using pf::pack_bf16;
using pf::rsrc;
using pf::Tile;
using pf::u32x2;

constexpr int kT = kPrefillThreads;
constexpr int kW = kT / kWave;  // waves per workgroup
constexpr int kL = 64;          // chunk tokens: one per lane

template <int R_, int P_, int N_>
struct TCfg {
  using T = bf16;
  using M = Mfma<bf16>;
  static constexpr int R = R_, P = P_, N = N_, NC = N_;
  static constexpr int es = 2;
  static constexpr int NPT = P_ / 16;          // p-tiles
  static constexpr int NNT = N_ / 16;          // n-tiles
  static constexpr int NPW = N_ / 2 / kW;      // rotation pairs per wave
  static constexpr int LR = kL * R_;           // rows of a chunk tile (token, rank)
  static constexpr int NQB = LR / 16;          // 16-row query (and key) blocks
  static constexpr int NTILES = NNT * NPT;     // 16 x 16 state tiles
  static constexpr int TPW = NTILES / kW;      // state tiles per wave
  // output units: one query block and PPG p-tiles; with few query blocks a
  // block's p-tiles are split over two units, so every wave has one
  static constexpr int PPG0 = (NQB * 2 <= kW && NPT >= 2) ? NPT / 2 : NPT;
  static constexpr int PPG = PPG0 < 4 ? PPG0 : 4;
  static constexpr int NPG = NPT / PPG;
  static constexpr int NOUT = NQB * NPG;
  // LDS of one ring buffer (bytes): B (then B~) and C (then C~) as [LR][N],
  // the weighted B~ as [LR][N], x as [LR][P], theta as [64][N/2] floats, dt
  // and lam of tokens u and u + 1 (4 x 64 floats), the per-token scalars
  // (cs, gamma, gamma + omega at a stride of kLMax floats), the chunk's
  // rotation per pair and the entry state [P][N] (bf16); then the
  // workgroup's words and the segment's rotation per pair
  static constexpr uint32_t kRowN = N_ * 2, kRowP = P_ * 2, kRowTh = N_ * 2;
  static constexpr uint32_t oB = 0;
  static constexpr uint32_t oC = oB + LR * kRowN;
  static constexpr uint32_t oW = oC + LR * kRowN;
  static constexpr uint32_t oX = oW + LR * kRowN;
  static constexpr uint32_t oTh = oX + LR * kRowP;
  static constexpr uint32_t oRaw = oTh + kL * kRowTh;
  static constexpr uint32_t oS = oRaw + 4 * kL * 4;
  static constexpr uint32_t oRot = oS + 3 * kLMax * 4;
  static constexpr uint32_t oG = oRot + (N_ / 2) * 8;
  static constexpr uint32_t kBuf = oG + P_ * kRowN;
  static constexpr int NBUF = 3;  // ring depth
  static constexpr uint32_t kMisc = 64 + (N_ / 2) * 8;
  static constexpr uint32_t oMisc = NBUF * kBuf;
  static constexpr uint32_t oSrot = oMisc + 64;
  static constexpr uint32_t kTotal = oMisc + kMisc;
  static constexpr bool kFits = kTotal <= kLdsLimit && NTILES % kW == 0 && TPW >= 1 &&
                                TPW <= kMaxStTiles && NPW >= 1 && PPG >= 1 &&
                                (kRowN == 128 || kRowN == 256) && (kRowP == 128 || kRowP == 256);
};

// Whether the layout fits (the ring in the LDS, whole state tiles per wave).
template <int R, int P, int N>
constexpr bool tok_fits() {
  return TCfg<R, P, N>::kFits;
}

// Tile of 16-byte columns XOR-swizzled by row (over up to 8 columns).
__device__ __forceinline__ Tile tile_at(unsigned char* base, uint32_t rowb) {
  const uint32_t ncol = rowb >> 4;
  return Tile{base, rowb, (ncol < 8u ? ncol : 8u) - 1u};
}

// NB bytes of v to a tile row at byte `byte` (16-byte pieces through the
// swizzle, smaller ones within one column).
template <int NB>
__device__ __forceinline__ void st_bytes(const Tile& t, uint32_t row, uint32_t byte,
                                         const uint32_t* v) {
  if constexpr (NB == 4) {
    t.ref<uint32_t>(row, byte) = v[0];
  } else if constexpr (NB == 8) {
    t.ref<u32x2>(row, byte) = u32x2{v[0], v[1]};
  } else {
    static_assert(NB % 16 == 0, "whole 16-byte vectors");
#pragma unroll
    for (int i = 0; i < NB / 16; ++i)
      t.ref<u32x4>(row, byte + 16 * i) = u32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
  }
}

// Uniform per-workgroup values.
struct TCtx {
  int b, h, bh, seg, c0, c1;
  uint32_t rowB, rowTh, rowDt, rowX;  // token strides in bytes
  float Ah;
};

typedef void __attribute__((address_space(3))) lds_void;
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

// Words of a raw buffer resource: base, no stride, `bytes` in range.
__device__ __forceinline__ u32x4v rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return u32x4v{(uint32_t)p, (uint32_t)(p >> 32) & 0xffffu, bytes, (uint32_t)pf::kRsrcWord3};
}

// LDS byte address of a pointer into the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const lds_void*)p);
}

// One direct global-to-LDS load: lane l's kBytes (4 or 16) at byte `voff` of
// the range land at LDS byte lds + kBytes l (zeros past the range).  Written
// as assembly because the compiler, which cannot tell which LDS bytes such a
// load writes, would otherwise make this wave's next LDS access wait for all
// of them; the caller orders the LDS instead: a barrier between the last
// read of a buffer and the loads into it, and s_waitcnt vmcnt, then a
// barrier, before the first read of what they bring.  M0 carries the LDS
// base (one wait state after its write) and is restored afterwards.
template <int kBytes>
__device__ __forceinline__ void dma_lds(u32x4v r, uint32_t lds, uint32_t voff) {
  uint32_t saved;
  if constexpr (kBytes == 16) {
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(voff), "s"(r)
        : "memory");
  } else {
    static_assert(kBytes == 4, "4 or 16 bytes a lane");
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "buffer_load_dword %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(voff), "s"(r)
        : "memory");
  }
}

// One 1 KB block of a row-major tile of `rowb`-byte rows (128 or 256) by a
// direct load: lane l fills slot l, i.e. row (row0 + l / cpr) and physical
// 16-byte column l % cpr, with the logical column that the tile's swizzle
// puts there; `gbyte(row)` is the row's byte offset in the buffer range.
template <uint32_t kRowb, class F>
__device__ __forceinline__ void lds_block(u32x4v r, unsigned char* tile, uint32_t row0, F gbyte) {
  constexpr uint32_t cpr = kRowb / 16;  // 16-byte columns per row
  constexpr uint32_t mask = (cpr < 8u ? cpr : 8u) - 1u;
  const uint32_t l = threadIdx.x & 63;
  const uint32_t row = row0 + l / cpr, pc = l % cpr;
  const uint32_t lc = pc ^ (row & mask);
  dma_lds<16>(r, lds_addr(tile + row0 * kRowb), gbyte(row) + lc * 16);
}

// Issue this wave's share of the direct loads of chunk c into ring buffer
// `buf`: the 1 KB blocks of B (and C), x and theta, dealt to the waves round
// robin, and (the last wave) dt and lam of tokens u and u + 1.  Returns nothing to
// wait for here: the caller waits (vmcnt) before the barrier that publishes
// the buffer.
template <class C, bool kWithC>
__device__ __forceinline__ void tok_issue(const PrefillArgs& a, const TCtx& s, int c,
                                          unsigned char* buf) {
  constexpr int R = C::R, N = C::N, P = C::P;
  const uint32_t w = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int t0 = c * kL;
  const int len = min(kL, a.T - t0);
  const size_t hrow = ((size_t)s.b * a.T + t0) * a.H + s.h;  // [B,T,H] row of token t0
  const uint32_t last = (uint32_t)(len - 1);
  constexpr uint32_t bcb = R * N * 2, xb = R * P * 2;
  // ranges end at the chunk's last valid byte: rows past the sequence land as 0
  const u32x4v rB =
      rsrc_words(static_cast<const unsigned char*>(a.B) + hrow * bcb, last * s.rowB + bcb);
  const u32x4v rX = rsrc_words(static_cast<const unsigned char*>(a.x) + hrow * xb, last * s.rowX + xb);
  const u32x4v rTh = a.theta ? rsrc_words(a.theta + hrow * (N / 2), last * s.rowTh + (N / 2) * 4)
                             : rsrc_words(nullptr, 0);
  const uint32_t rowB = s.rowB, rowX = s.rowX, rowTh = s.rowTh;
  // B and C rows are (token, rank): token u = row / R, rank row % R
  auto gB = [rowB](uint32_t row) { return (row / R) * rowB + (row % R) * (N * 2); };
  auto gX = [rowX](uint32_t row) { return (row / R) * rowX + (row % R) * (P * 2); };
  auto gT = [rowTh](uint32_t row) { return row * rowTh; };
  constexpr uint32_t kBlkN = C::LR * C::kRowN / 1024, kRowsN = 1024 / C::kRowN;
  constexpr uint32_t kBlkX = C::LR * C::kRowP / 1024, kRowsX = 1024 / C::kRowP;
  constexpr uint32_t kBlkT = kL * C::kRowTh / 1024, kRowsT = 1024 / C::kRowTh;
  for (uint32_t j = w; j < kBlkN; j += kW)
    lds_block<C::kRowN>(rB, buf + C::oB, j * kRowsN, gB);
  if constexpr (kWithC) {
    const u32x4v rC =
        rsrc_words(static_cast<const unsigned char*>(a.C) + hrow * bcb, last * s.rowB + bcb);
    for (uint32_t j = w; j < kBlkN; j += kW)
      lds_block<C::kRowN>(rC, buf + C::oC, j * kRowsN, gB);
  }
  for (uint32_t j = w; j < kBlkX; j += kW)
    lds_block<C::kRowP>(rX, buf + C::oX, j * kRowsX, gX);
  for (uint32_t j = w; j < kBlkT; j += kW)
    lds_block<C::kRowTh>(rTh, buf + C::oTh, j * kRowsT, gT);
  if (w == kW - 1) {
    // dt and lam of token u, and of token u + 1 (its omega needs the token
    // after the chunk), up to the sequence's end
    const uint32_t u = threadIdx.x & 63;
    const int nsc = min(kL + 1, a.T - t0);
    const uint32_t scb = (uint32_t)(nsc - 1) * s.rowDt + 4;
    const u32x4v rD = rsrc_words(a.dt + hrow, scb);
    const uint32_t raw = lds_addr(buf + C::oRaw);
    dma_lds<4>(rD, raw, u * s.rowDt);
    dma_lds<4>(rD, raw + 256, (u + 1) * s.rowDt);
    if (a.lam) {
      const u32x4v rL = rsrc_words(a.lam + hrow, scb);
      dma_lds<4>(rL, raw + 512, u * s.rowDt);
      dma_lds<4>(rL, raw + 768, (u + 1) * s.rowDt);
    }
  }
}

// The buffers of one chunk step.
struct TBuf {
  unsigned char* base;
  Tile B, C, W, X, Th, G;
  float* raw;    // dt, dt of the next token, lam, lam of the next token (64 each)
  float* sc;     // cs, gamma, gamma + omega (stride kLMax)
  float2* rot;   // (cos, sin) of the chunk's total angle per pair
};

template <class C>
__device__ __forceinline__ TBuf tok_buf(unsigned char* smem, int bb) {
  // the base offset is made opaque so that per-lane addresses are formed in
  // each step rather than kept live across the chunk loop
  unsigned char* base = smem + pf::opaque_u((uint32_t)bb * C::kBuf);
  TBuf t;
  t.base = base;
  t.B = tile_at(base + C::oB, C::kRowN);
  t.C = tile_at(base + C::oC, C::kRowN);
  t.W = tile_at(base + C::oW, C::kRowN);
  t.X = tile_at(base + C::oX, C::kRowP);
  t.Th = tile_at(base + C::oTh, C::kRowTh);
  t.G = tile_at(base + C::oG, C::kRowN);
  t.raw = reinterpret_cast<float*>(base + C::oRaw);
  t.sc = reinterpret_cast<float*>(base + C::oS);
  t.rot = reinterpret_cast<float2*>(base + C::oRot);
  return t;
}

// NB bytes of a tile row at byte `byte` into v (16-byte pieces through the
// swizzle).
template <int NB>
__device__ __forceinline__ void ld_tile(const Tile& t, uint32_t row, uint32_t byte, uint32_t* v) {
  static_assert(NB % 16 == 0, "whole 16-byte vectors");
#pragma unroll
  for (int i = 0; i < NB / 16; ++i) {
    const u32x4 q = t.ref<u32x4>(row, byte + 16 * i);
    v[4 * i] = q[0];
    v[4 * i + 1] = q[1];
    v[4 * i + 2] = q[2];
    v[4 * i + 3] = q[3];
  }
}

// Rotation step of one chunk for this lane (token u) and wave (its pairs),
// from the staged raw inputs of buffer t: per-token scalars, chunk-local
// angles, B (and C) rotated in place, the weighted B~, the chunk's rotation
// per pair.  Returns the
// chunk's log-decay cs_e; the lanes below NPW add their pair's chunk angle
// (revolutions, reduced) to sang.
template <class C, bool kOut>
__device__ __forceinline__ float tok_rotate(const TBuf& t, bool has_lam, float Ah,
                                            double& sang) {
  constexpr int R = C::R, NPW = C::NPW;
  const uint32_t u = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float d = t.raw[u], dn = t.raw[64 + u];
  // without lam the weight is 1 (the exponential-Euler rule)
  const float l = has_lam ? t.raw[128 + u] : 1.f, ln = has_lam ? t.raw[192 + u] : 1.f;
  uint32_t th[NPW];
  ld_tile<NPW * 4>(t.Th, u, w * (NPW * 4), th);
  // per-token scalars (exponential-trapezoidal weights; every wave has them)
  const float cs = wave_incl_scan(d * Ah);
  const float cse = wave_read_lane(cs, 63);
  const float ga = l * d;
  const float gom = ga + (1.f - ln) * dn;
  const float wgt = __expf(cse - cs) * gom;
  if (kOut && w == 0) {
    t.sc[u] = cs;
    t.sc[kLMax + u] = ga;
    t.sc[2 * kLMax + u] = gom;
  }
  // chunk-local cumulative angles in revolutions: in-row scan of values
  // reduced to [0, 1), reduced again, then the cross-row steps
  const float dr = d * kInv2Pi;
  float ph[NPW];
#pragma unroll
  for (int k = 0; k < NPW; ++k) ph[k] = __builtin_amdgcn_fractf(dr * __uint_as_float(th[k]));
#pragma unroll
  for (int k = 0; k < NPW; ++k) ph[k] += dpp_move<0x111>(ph[k]);  // row_shr:1
#pragma unroll
  for (int k = 0; k < NPW; ++k) ph[k] += dpp_move<0x112>(ph[k]);  // row_shr:2
#pragma unroll
  for (int k = 0; k < NPW; ++k) ph[k] += dpp_move<0x114>(ph[k]);  // row_shr:4
#pragma unroll
  for (int k = 0; k < NPW; ++k) ph[k] = __builtin_amdgcn_fractf(ph[k] + dpp_move<0x118>(ph[k]));
#pragma unroll
  for (int k = 0; k < NPW; ++k) ph[k] += dpp_move<0x142, 0xa>(ph[k]);  // row_bcast:15
#pragma unroll
  for (int k = 0; k < NPW; ++k) ph[k] += dpp_move<0x143, 0xc>(ph[k]);  // row_bcast:31
  // the chunk's total angle per pair (lane 63), to lane k for pair k
  float mine = 0.f;
#pragma unroll
  for (int k = 0; k < NPW; ++k) {
    const float tot = wave_read_lane(ph[k], 63);
    mine = u == (uint32_t)k ? tot : mine;
  }
  // the rotation R(phi)^T of a pair (b0, b1) is (c b0 + s b1, c b1 - s b0):
  // two bf16 dot products of the stored pair with (c, s) and (-s, c), whose
  // products are exact in fp32 (the inputs are bf16 already; c and s are
  // rounded to bf16, as the rotated values are when they are stored)
  bf16x2 rcs[NPW], rncs[NPW];
#pragma unroll
  for (int k = 0; k < NPW; ++k) {
    const float sn = __builtin_amdgcn_sinf(ph[k]), cn = __builtin_amdgcn_cosf(ph[k]);
    rcs[k] = bf16x2{from_f32<bf16>(cn), from_f32<bf16>(sn)};
    rncs[k] = bf16x2{from_f32<bf16>(-sn), from_f32<bf16>(cn)};
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t row = u * R + r;
    uint32_t bv[NPW], cv[NPW], bw[NPW], bt[NPW], ct[NPW];
    ld_tile<NPW * 4>(t.B, row, w * (NPW * 4), bv);
    if constexpr (kOut) ld_tile<NPW * 4>(t.C, row, w * (NPW * 4), cv);
#pragma unroll
    for (int k = 0; k < NPW; ++k) {
      const bf16x2 bp = __builtin_bit_cast(bf16x2, bv[k]);
      const float rb0 = __builtin_amdgcn_fdot2_f32_bf16(bp, rcs[k], 0.f, false);
      const float rb1 = __builtin_amdgcn_fdot2_f32_bf16(bp, rncs[k], 0.f, false);
      bw[k] = pack_bf16(wgt * rb0, wgt * rb1);
      if constexpr (kOut) {
        bt[k] = pack_bf16(rb0, rb1);
        const bf16x2 cp = __builtin_bit_cast(bf16x2, cv[k]);
        ct[k] = pack_bf16(__builtin_amdgcn_fdot2_f32_bf16(cp, rcs[k], 0.f, false),
                          __builtin_amdgcn_fdot2_f32_bf16(cp, rncs[k], 0.f, false));
      }
    }
    // B~ and C~ in place (for the scores), the weighted B~ into its tile
    st_bytes<NPW * 4>(t.W, row, w * (NPW * 4), bw);
    if constexpr (kOut) {
      st_bytes<NPW * 4>(t.B, row, w * (NPW * 4), bt);
      st_bytes<NPW * 4>(t.C, row, w * (NPW * 4), ct);
    }
  }
  // the chunk's rotation (fp32 sine and cosine of the total angle reduced to
  // half a revolution either side of zero), and the segment's angle summed
  // in double
  if (u < (uint32_t)NPW) {
    const float f = mine - __builtin_rintf(mine);
    t.rot[w * NPW + u] = make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
    sang += static_cast<double>(f);
    sang -= __builtin_rint(sang);
  }
  return cse;
}

// Entry state of the chunk into the tile [P][N] (bf16), from this wave's
// state tiles (tile i = wave + kW m: n-tile i % NNT, p-tile i / NNT; lane
// (g, c) holds rows 4g..4g+3 of column c).
template <class C>
__device__ __forceinline__ void tok_state_to_lds(const f32x4 (&stt)[kMaxStTiles], const Tile& tG) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
#pragma unroll
  for (int m = 0; m < C::TPW; ++m) {
    const int i = wave + kW * m;
    const int nt = i % C::NNT, pt = i / C::NNT;
    tG.ref<u32x2>((uint32_t)(pt * 16 + li), (uint32_t)((nt * 16 + 4 * g) * 2)) =
        u32x2{pack_bf16(stt[m][0], stt[m][1]), pack_bf16(stt[m][2], stt[m][3])};
  }
}

// MFMA fragment read straight from a row-major tile whose row is the
// contraction: lane (g, i) gets row `row`, slots k0 + 8g .. k0 + 8g + 7.
__device__ __forceinline__ bf16x8 frag_row(const Tile& t, uint32_t row, int k0) {
  const int g = (threadIdx.x & 63) >> 4;
  return t.ref2<bf16x8>(row, 16u * g, (uint32_t)k0 * 2u);
}

typedef bf16x4 __attribute__((address_space(3))) lds_bf16x4;

// MFMA fragment of a row-major tile whose rows are the contraction, through
// two LDS transpose reads: lane (g, i) gets column 16 ctile + i of rows r0 ..
// r0 + 3 (slots 0..3) and r1 .. r1 + 3 (slots 4..7), where r0 and r1 may
// depend on g.  In each read, source lane s of a 16-lane group reads the 8
// bytes of row r + s / 4 at columns 16 ctile + 4 (s % 4) .. + 3; the
// transpose hands lane i element i % 4 of the reads of lanes i / 4 + 4 m,
// m = 0..3, i.e. column 16 ctile + i of rows r .. r + 3.
__device__ __forceinline__ bf16x8 frag_tr(const Tile& t, uint32_t r0, uint32_t r1, int ctile) {
  const uint32_t s = threadIdx.x & 15;
  const uint32_t byte = 32u * (uint32_t)ctile + 8u * (s & 3u);
  const lds_bf16x4* p0 = (const lds_bf16x4*)(t.base + t.at(r0 + (s >> 2), byte));
  const lds_bf16x4* p1 = (const lds_bf16x4*)(t.base + t.at(r1 + (s >> 2), byte));
  const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<lds_bf16x4*>(p0));
  const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<lds_bf16x4*>(p1));
  return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Chunk state of this wave's tiles, S = sum over rows of Bw^T X (A from the
// weighted B~ tile, B from the x tile, both through transpose reads), folded
// in: stt <- R(Phi_c)(d stt + S).
template <class C>
__device__ __forceinline__ void tok_state_update(const TBuf& t, float d,
                                                 f32x4 (&stt)[kMaxStTiles]) {
  using M = typename C::M;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  // every tile of a wave has the same n-tile (kW is a multiple of NNT or
  // NNT of kW): one A fragment serves all
  const int nt = wave % C::NNT;
  f32x4 acc[C::TPW];
#pragma unroll
  for (int m = 0; m < C::TPW; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k0 = 0; k0 < C::LR; k0 += M::K) {
    const uint32_t r0 = (uint32_t)(k0 + 8 * g);
    const bf16x8 fa = frag_tr(t.W, r0, r0 + 4, nt);
#pragma unroll
    for (int m = 0; m < C::TPW; ++m) {
      const int pt = (wave + kW * m) / C::NNT;
      acc[m] = M::mma(fa, frag_tr(t.X, r0, r0 + 4, pt), acc[m]);
    }
  }
  // rows 4g .. 4g + 3 of n-tile nt: pairs 8 nt + 2g and 8 nt + 2g + 1
  const float2 q0 = t.rot[nt * 8 + 2 * g], q1 = t.rot[nt * 8 + 2 * g + 1];
#pragma unroll
  for (int m = 0; m < C::TPW; ++m) {
    const float v0 = d * stt[m][0] + acc[m][0], v1 = d * stt[m][1] + acc[m][1];
    const float v2 = d * stt[m][2] + acc[m][2], v3 = d * stt[m][3] + acc[m][3];
    stt[m][0] = q0.x * v0 - q0.y * v1;
    stt[m][1] = q0.y * v0 + q0.x * v1;
    stt[m][2] = q1.x * v2 - q1.y * v3;
    stt[m][3] = q1.y * v2 + q1.x * v3;
  }
}

// One output unit, computed transposed: y^T rows p (PPG p-tiles from p_lo)
// by the 16 query rows of block qb.
//   y_t = exp(cs_t) C~_t^T G + sum_u W[t,u] (C~_t^T B~_u) x_u^T
// with W the chunk's decay x 2-band trapezoid mask (Mamba-3 paper
// translation, section 3.1, equation 7): the inter-chunk term is G^T C~^T,
// the scores S^T = B~ C~^T (keys x queries) are masked in registers, and
// their accumulator layout is the B operand of the product with x^T.
template <class C>
__device__ __forceinline__ void tok_output_unit(const TBuf& t, const rsrc& ry, uint32_t rowX,
                                                int qb, int p_lo) {
  using M = typename C::M;
  constexpr int R = C::R, P = C::P, N = C::N, PPG = C::PPG;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const uint32_t qrow = (uint32_t)(qb * 16 + li);
  const int tq = (qb * 16 + li) / R;
  const float csq = t.sc[tq];
  f32x4 acc[PPG];
#pragma unroll
  for (int pp = 0; pp < PPG; ++pp) acc[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
  // inter-chunk term, then every column (query) scaled by exp(cs_q)
#pragma unroll
  for (int n0 = 0; n0 < N; n0 += M::K) {
    const bf16x8 fq = frag_row(t.C, qrow, n0);
#pragma unroll
    for (int pp = 0; pp < PPG; ++pp)
      acc[pp] = M::mma(frag_row(t.G, (uint32_t)((p_lo + pp) * 16 + li), n0), fq, acc[pp]);
  }
  const float eq = __expf(csq);
#pragma unroll
  for (int pp = 0; pp < PPG; ++pp)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[pp][j] *= eq;
  // intra-chunk term over pairs of 16-row key blocks up to the diagonal
  for (int kb = 0; kb <= qb; kb += 2) {
    f32x4 sct[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int n0 = 0; n0 < N; n0 += M::K) {
      const bf16x8 fq = frag_row(t.C, qrow, n0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        sct[i] = M::mma(frag_row(t.B, (uint32_t)((kb + i) * 16 + li), n0), fq, sct[i]);
    }
    float kcs[2][4], kga[2][4], kgom[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      pf::key_scalars4<R>(t.sc, (kb + i) * 16 + 4 * g, kcs[i], kga[i], kgom[i]);
    pf::mask_scores<R, 2>(sct, kcs, kga, kgom, kb, g, tq, csq);
    bf16x8 fs;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      fs[j] = from_f32<bf16>(sct[0][j]);
      fs[4 + j] = from_f32<bf16>(sct[1][j]);
    }
    // x^T with the scores' slot order: keys 16 kb + 4g .. + 3, then 16 (kb +
    // 1) + 4g .. + 3
    const uint32_t r0 = (uint32_t)(kb * 16 + 4 * g), r1 = r0 + 16;
#pragma unroll
    for (int pp = 0; pp < PPG; ++pp) acc[pp] = M::mma(frag_tr(t.X, r0, r1, p_lo + pp), fs, acc[pp]);
  }
  // lane (g, c): p = 16 (p_lo + pp) + 4g .. + 3 of query row qb * 16 + c
  const uint32_t q = qrow;
  const uint32_t ob = (q / R) * rowX + (q % R) * (P * 2);
#pragma unroll
  for (int pp = 0; pp < PPG; ++pp) {
    const uint32_t o = ob + (uint32_t)(((p_lo + pp) * 16 + 4 * g) * 2);
    const u32x2 v = {pack_bf16(acc[pp][0], acc[pp][1]), pack_bf16(acc[pp][2], acc[pp][3])};
    __builtin_amdgcn_raw_buffer_store_b64(v, ry, (int)o, 0, 0);
  }
}

// y of one chunk: units (query block, p-group) dealt to the waves w, 2kW-1-w,
// 2kW+w, ... so the causal (growing) cost per query block balances.
template <class C>
__device__ __forceinline__ void tok_outputs(const PrefillArgs& a, const TCtx& s, int c,
                                            const TBuf& t) {
  const int wave = threadIdx.x >> 6;
  const int t0 = c * kL;
  const int len = min(kL, a.T - t0);
  const size_t hrow = ((size_t)s.b * a.T + t0) * a.H + s.h;
  constexpr uint32_t yb = C::R * C::P * 2;
  const rsrc ry = make_rsrc(static_cast<unsigned char*>(a.y) + hrow * yb,
                            (uint32_t)(len - 1) * s.rowX + yb);
#pragma unroll
  for (int k = 0; k * kW < C::NOUT; ++k) {
    const int unit = (k & 1) ? (k + 1) * kW - 1 - wave : k * kW + wave;
    if (unit < C::NOUT)
      tok_output_unit<C>(t, ry, s.rowX, unit / C::NPG, (unit % C::NPG) * C::PPG);
  }
}

template <class C>
__device__ __forceinline__ void tok_segment(const PrefillArgs& a, int ticket,
                                            unsigned char* smem) {
  constexpr int NB = C::NBUF;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int BH = a.nb * a.H;
  TCtx s;
  s.seg = ticket / BH;
  s.bh = ticket % BH;
  s.b = s.bh / a.H;
  s.h = s.bh % a.H;
  s.c0 = s.seg * a.K;
  s.c1 = min(a.nC, s.c0 + a.K);
  s.rowB = (uint32_t)(a.H * C::R * C::N * 2);
  s.rowTh = (uint32_t)(a.H * (C::N / 2) * 4);
  s.rowDt = (uint32_t)(a.H * 4);
  s.rowX = (uint32_t)(a.H * C::R * C::P * 2);
  // a uniform value, taken into a scalar register here so that its load is
  // complete before the chunk loop
  s.Ah = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.A[s.h])));
  const bool has_lam = a.lam != nullptr;
  int* s_misc = reinterpret_cast<int*>(smem + C::oMisc);
  float2* s_srot = reinterpret_cast<float2*>(smem + C::oSrot);

  // The segment is a sequence of 2K items: the local pass over its K chunks,
  // then the output pass over them again.  Item i lives in ring buffer i % NB.
  const int K = s.c1 - s.c0;
  const int nitem = 2 * K;
  auto issue = [&](int i) {
    if (i >= nitem) return;
    unsigned char* buf = smem + (uint32_t)(i % NB) * C::kBuf;
    if (i < K)
      tok_issue<C, false>(a, s, s.c0 + i, buf);
    else
      tok_issue<C, true>(a, s, s.c0 + i - K, buf);
  };

  f32x4 stt[kMaxStTiles];
#pragma unroll
  for (int q = 0; q < kMaxStTiles; ++q) stt[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  double sang = 0.0;  // lanes < NPW: the segment's angle of pair wave * NPW + lane
  float seg_logdecay = 0.f;

  // prologue: item 0 staged and published, item 1 on its way
  issue(0);
  __builtin_amdgcn_s_waitcnt(0);
  issue(1);
  __syncthreads();

  for (int i = 0; i < nitem; ++i) {
    const bool local = i < K;
    const int c = local ? s.c0 + i : s.c0 + i - K;
    const TBuf t = tok_buf<C>(smem, i % NB);
    float cse;
    if (local) {
      cse = tok_rotate<C, false>(t, has_lam, s.Ah, sang);
    } else {
      double unused = 0.0;
      cse = tok_rotate<C, true>(t, has_lam, s.Ah, unused);
      tok_state_to_lds<C>(stt, t.G);
    }
    // the next item's loads (issued a step ago) have landed
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (!local) tok_outputs<C>(a, s, c, t);
    tok_state_update<C>(t, __expf(cse), stt);
    // the buffer of item i + NB - 1 was last read in the previous step's
    // MFMA phase, which every wave finished before this step's barrier.  Its
    // loads go out after this step's own LDS-heavy MFMA work (issued at the
    // barrier they competed with it: 58.7 against 55.0 us on the SISO bench
    // shape) and still have the next step to land; at the end of the local
    // pass they fly during the chain (issued after it: 58.8 us)
    issue(i + NB - 1);
    if (local) seg_logdecay += cse;
    if (i == K - 1) {
      // ---- between the passes: the chain (chain_phase) -------------------
      if (lane < C::NPW) {
        const float f = static_cast<float>(sang);
        s_srot[(tid >> 6) * C::NPW + lane] =
            make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
      }
      __syncthreads();  // s_srot; every MFMA read of the local pass is done
      const WaveRoles wr = {0, 0, 0, 0, kW};
      f32x4 ent[kMaxStTiles];
      pf::chain_phase<C>(a, wr, s.seg, s.bh, ticket, __expf(seg_logdecay), s_srot, s_misc, stt,
                         ent);
#pragma unroll
      for (int q = 0; q < kMaxStTiles; ++q) stt[q] = ent[q];
      // every load of the chain has returned: otherwise a load whose value
      // the chain did not need leaves the compiler a pending write to its
      // register, and it would wait for all memory at the top of every step
      __builtin_amdgcn_s_waitcnt(0);
    }
  }
}

template <class C>
__global__ void __launch_bounds__(kT) prefill_tok_kernel(PrefillArgs a_in) {
  extern __shared__ __align__(16) unsigned char smem[];
  PrefillArgs a = a_in;
  a.N = C::N;
  int* s_misc = reinterpret_cast<int*>(smem + C::oMisc);
  const int ticket = pf::take_ticket(a, s_misc);
  if (ticket >= 0 && ticket < (int)gridDim.x)
    tok_segment<C>(a, ticket, smem);
  else
    pf::bad_ticket(a);
  pf::finish_workgroup(a, s_misc);
}

template <class C>
hipError_t launch_tok(const PrefillArgs& a, hipStream_t stream) {
  const hipError_t attr = lds_limit(reinterpret_cast<const void*>(&prefill_tok_kernel<C>), C::kTotal);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((prefill_tok_kernel<C>), dim3(a.nb * a.H * a.nSeg), dim3(kT), C::kTotal,
                     stream, a);
  return hipGetLastError();
}

}  // namespace pt
}  // namespace m3

namespace m3 {
namespace pt {

// Launch the token-lane kernel for rank R if it takes the shape (N and P
// fixed at compile time); *taken says whether it did.
template <int R, int P, int N>
hipError_t try_tok(const PrefillArgs& a, hipStream_t stream, bool* taken) {
  if constexpr (tok_fits<R, P, N>()) {
    *taken = true;
    return launch_tok<TCfg<R, P, N>>(a, stream);
  } else {
    *taken = false;
    return hipSuccess;
  }
}

// The shapes the token-lane kernel takes: bfloat16, rank 1, 64-token chunks,
// state size 64 and head dimension 64 (where its ring fits the LDS).
inline hipError_t tok_dispatch(const PrefillArgs& a, hipStream_t stream, bool* taken) {
  *taken = false;
  if (a.L != kL || a.R != 1 || a.N != 64 || a.P != 64) return hipSuccess;
  return try_tok<1, 64, 64>(a, stream, taken);
}

}  // namespace pt
}  // namespace m3
