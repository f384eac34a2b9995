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
//
// Two kernels share this layout.  prefill_tok_kernel walks a segment twice
// (a local pass for its exit state, then the output pass from the true entry
// state), like prefill_impl.h.  prefill_tok1_kernel, for segments of up to
// eight chunks (the segment rule gives eight at the SISO bench shape), walks
// it once: each chunk's outputs are computed from the segment's zero-entry
// state, C~ and the scalars stay in the LDS and the partial outputs in
// registers, and after the chain a correction adds the entry state's share
// exp(cs_t) C~_t^T E_c (the state is linear in its entry), so no input is
// read or rotated twice.  See tok1_segment.
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
  static constexpr int kAggBatch = N_ == 64 ? pf::kBatch : pf::kBatch / 2;  // chain look-back
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
  // The single pass (tok1_segment, segments of at most kK1 chunks): a ring
  // of three staging buffers (B, then B~; x; theta; dt and lam of the
  // chunk's tokens and the token after it), two buffers of computed values
  // (the entry state [P][N] the outputs see; gamma, gamma + omega and the
  // state weight per token), and per chunk of the segment, kept to its end:
  // C (then C~), the log-decay prefix cs and the chunk's angle per pair.
  // The correction's entry-state tiles reuse the ring.
  static constexpr int kK1 = 8;
  static constexpr uint32_t o1B = 0;
  static constexpr uint32_t o1X = o1B + LR * kRowN;
  static constexpr uint32_t o1Th = o1X + LR * kRowP;
  static constexpr uint32_t o1Raw = o1Th + kL * kRowTh;
  static constexpr uint32_t k1Sc = (kL + 4) * 4;  // 65 floats, padded
  static constexpr uint32_t k1Ring = o1Raw + 2 * k1Sc;
  static constexpr uint32_t o1Dbl = 3 * k1Ring;
  static constexpr uint32_t o1G = 0;
  static constexpr uint32_t o1Gs = o1G + P_ * kRowN;
  static constexpr uint32_t k1Dbl = o1Gs + 3 * kL * 4;
  static constexpr uint32_t o1Per = o1Dbl + 2 * k1Dbl;
  static constexpr uint32_t o1C = 0;
  static constexpr uint32_t o1Cs = o1C + LR * kRowN;
  static constexpr uint32_t o1Ang = o1Cs + kL * 4;
  static constexpr uint32_t k1Per = o1Ang + (N_ / 2) * 4;
  static constexpr uint32_t o1Misc = o1Per + kK1 * k1Per;
  static constexpr uint32_t o1Srot = o1Misc + 64;
  static constexpr uint32_t k1Total = o1Misc + kMisc;
  // one output unit per wave (its partial outputs stay in its registers),
  // rank 1, and the correction's kK1 entry-state tiles fit the ring
  static constexpr bool k1Fits = kFits && k1Total <= kLdsLimit && NOUT == kW && R_ == 1 &&
                                 kK1 * P_ * kRowN <= 3 * k1Ring;
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
// Where one chunk's staged inputs land: the B, C, x and theta tiles and the
// raw dt / lam words (each may lie in a different LDS area).
struct TDst {
  unsigned char *B, *C, *X, *Th, *raw;
};

template <class C, bool kWithC, bool kCompact = false>
__device__ __forceinline__ void tok_issue(const PrefillArgs& a, const TCtx& s, int c,
                                          const TDst& d) {
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
    lds_block<C::kRowN>(rB, d.B, j * kRowsN, gB);
  if constexpr (kWithC) {
    const u32x4v rC =
        rsrc_words(static_cast<const unsigned char*>(a.C) + hrow * bcb, last * s.rowB + bcb);
    for (uint32_t j = w; j < kBlkN; j += kW)
      lds_block<C::kRowN>(rC, d.C, j * kRowsN, gB);
  }
  for (uint32_t j = w; j < kBlkX; j += kW)
    lds_block<C::kRowP>(rX, d.X, j * kRowsX, gX);
  for (uint32_t j = w; j < kBlkT; j += kW)
    lds_block<C::kRowTh>(rTh, d.Th, j * kRowsT, gT);
  if (w == kW - 1) {
    // dt and lam of token u, and of token u + 1 (its omega needs the token
    // after the chunk), up to the sequence's end
    const uint32_t u = threadIdx.x & 63;
    const int nsc = min(kL + 1, a.T - t0);
    const uint32_t scb = (uint32_t)(nsc - 1) * s.rowDt + 4;
    const u32x4v rD = rsrc_words(a.dt + hrow, scb);
    const uint32_t raw = lds_addr(d.raw);
    if constexpr (kCompact) {
      // tokens 0..63, then token 64 by lane 0 alone (its word lands at
      // float 64): 65 floats of dt, then of lam at float 68
      dma_lds<4>(rD, raw, u * s.rowDt);
      if (u == 0) dma_lds<4>(rD, raw + 256, 64 * s.rowDt);
      if (a.lam) {
        const u32x4v rL = rsrc_words(a.lam + hrow, scb);
        dma_lds<4>(rL, raw + C::k1Sc, u * s.rowDt);
        if (u == 0) dma_lds<4>(rL, raw + C::k1Sc + 256, 64 * s.rowDt);
      } else {
        // without lam the weight is 1 (the exponential-Euler rule): ones
        // in its place, so the rotation reads lam on every path (the
        // barrier after this step orders these stores before it)
        float* lw = reinterpret_cast<float*>(d.raw + C::k1Sc);
        lw[u] = 1.f;
        if (u == 0) lw[64] = 1.f;
      }
    } else {
      dma_lds<4>(rD, raw, u * s.rowDt);
      dma_lds<4>(rD, raw + 256, (u + 1) * s.rowDt);
      if (a.lam) {
        const u32x4v rL = rsrc_words(a.lam + hrow, scb);
        dma_lds<4>(rL, raw + 512, u * s.rowDt);
        dma_lds<4>(rL, raw + 768, (u + 1) * s.rowDt);
      }
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
  // the single pass: raw holds 65 floats of dt, then of lam (stride k1Sc);
  // cs (64 floats), gamma, gamma + omega and the state weight (stride 64),
  // the chunk's angle per pair in revolutions
  float *cs, *gs, *ang;
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
// kSplit (the single pass, with kOut): the raw words are 65 floats of dt and
// of lam; the scalars go to t.cs and t.gs (with the state weight, which the
// state update applies to its operand instead of a weighted B~ tile) and
// the chunk's angle to t.ang.
template <class C, bool kOut, bool kSplit = false>
__device__ __forceinline__ float tok_rotate(const TBuf& t, bool has_lam, float Ah,
                                            double& sang) {
  constexpr int R = C::R, NPW = C::NPW;
  static_assert(!kSplit || kOut, "the single pass rotates B and C");
  const uint32_t u = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr uint32_t kLam = kSplit ? C::k1Sc / 4 : 128, kNext = kSplit ? 1 : 64;
  const float d = t.raw[u], dn = t.raw[kNext + u];
  // without lam the weight is 1 (the exponential-Euler rule); the single
  // pass stages ones then, and reads lam on every path
  const float l = (kSplit || has_lam) ? t.raw[kLam + u] : 1.f;
  const float ln = (kSplit || has_lam) ? t.raw[kLam + kNext + u] : 1.f;
  uint32_t th[NPW];
  ld_tile<NPW * 4>(t.Th, u, w * (NPW * 4), th);
  // this lane's pairs of B (and C), requested with the other reads, before
  // the scalar stores below, which the compiler would not move them across
  uint32_t bv[R][NPW], cv[R][NPW];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    ld_tile<NPW * 4>(t.B, u * R + r, w * (NPW * 4), bv[r]);
    if constexpr (kOut) ld_tile<NPW * 4>(t.C, u * R + r, w * (NPW * 4), cv[r]);
  }
  // per-token scalars (exponential-trapezoidal weights; every wave has them)
  const float cs = wave_incl_scan(d * Ah);
  const float cse = wave_read_lane(cs, 63);
  const float ga = l * d;
  const float gom = ga + (1.f - ln) * dn;
  const float wgt = __expf(cse - cs) * gom;
  if constexpr (kSplit) {
    if (w == 0) {
      t.cs[u] = cs;
      t.gs[u] = ga;
      t.gs[kL + u] = gom;
      t.gs[2 * kL + u] = wgt;
    }
  } else if (kOut && w == 0) {
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
    uint32_t bw[NPW], bt[NPW], ct[NPW];
#pragma unroll
    for (int k = 0; k < NPW; ++k) {
      const bf16x2 bp = __builtin_bit_cast(bf16x2, bv[r][k]);
      const float rb0 = __builtin_amdgcn_fdot2_f32_bf16(bp, rcs[k], 0.f, false);
      const float rb1 = __builtin_amdgcn_fdot2_f32_bf16(bp, rncs[k], 0.f, false);
      if constexpr (!kSplit) bw[k] = pack_bf16(wgt * rb0, wgt * rb1);
      if constexpr (kOut) {
        bt[k] = pack_bf16(rb0, rb1);
        const bf16x2 cp = __builtin_bit_cast(bf16x2, cv[r][k]);
        ct[k] = pack_bf16(__builtin_amdgcn_fdot2_f32_bf16(cp, rcs[k], 0.f, false),
                          __builtin_amdgcn_fdot2_f32_bf16(cp, rncs[k], 0.f, false));
      }
    }
    // B~ and C~ in place (for the scores), the weighted B~ into its tile
    if constexpr (!kSplit) st_bytes<NPW * 4>(t.W, row, w * (NPW * 4), bw);
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
    if constexpr (kSplit)
      t.ang[w * NPW + u] = f;
    else
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

// Inter-chunk term of one output unit, computed transposed (y^T rows p:
// PPG p-tiles from p_lo, by the query row of this lane's column):
// acc += exp(cs_q) G^T C~_q, G the state a chunk's outputs see (as a [P][N]
// tile) and C~ the chunk's rotated C.
template <class C>
__device__ __forceinline__ void tok_inter(const Tile& G, const Tile& Cq, uint32_t qrow, int p_lo,
                                          float eq, f32x4 (&acc)[C::PPG]) {
  using M = typename C::M;
  constexpr int N = C::N, PPG = C::PPG;
  const int li = threadIdx.x & 15;
  f32x4 t[PPG];
#pragma unroll
  for (int pp = 0; pp < PPG; ++pp) t[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int n0 = 0; n0 < N; n0 += M::K) {
    const bf16x8 fq = frag_row(Cq, qrow, n0);
#pragma unroll
    for (int pp = 0; pp < PPG; ++pp)
      t[pp] = M::mma(frag_row(G, (uint32_t)((p_lo + pp) * 16 + li), n0), fq, t[pp]);
  }
#pragma unroll
  for (int pp = 0; pp < PPG; ++pp)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[pp][j] = __builtin_fmaf(t[pp][j], eq, acc[pp][j]);
}

// Intra-chunk term of one output unit (query block qb, PPG p-tiles from
// p_lo), added to acc:
//   y_t += sum_u W[t,u] (C~_t^T B~_u) x_u^T
// with W the chunk's decay x 2-band trapezoid mask (Mamba-3 paper
// translation, section 3.1, equation 7).  The scores S^T = B~ C~^T (keys x
// queries) are masked in registers, and their accumulator layout is the B
// operand of the product with x^T.
template <class C>
__device__ __forceinline__ void tok_intra(const TBuf& t, int qb, int p_lo, f32x4 (&acc)[C::PPG]) {
  using M = typename C::M;
  constexpr int R = C::R, N = C::N, PPG = C::PPG;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const uint32_t qrow = (uint32_t)(qb * 16 + li);
  const int tq = (qb * 16 + li) / R;
  const float csq = t.sc[tq];
  // over pairs of 16-row key blocks up to the diagonal
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
}

// y of one output unit from its accumulators: lane (g, c) holds p = 16
// (p_lo + pp) + 4g .. + 3 of query row qb * 16 + c, stored as one 8-byte
// vector per p-tile (lanes past the sequence's end are dropped by the range).
template <class C>
__device__ __forceinline__ void tok_unit_store(const rsrc& ry, uint32_t rowX, int qb, int p_lo,
                                               const f32x4 (&acc)[C::PPG]) {
  constexpr int R = C::R, P = C::P;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const uint32_t q = (uint32_t)(qb * 16 + li);
  const uint32_t ob = (q / R) * rowX + (q % R) * (P * 2);
#pragma unroll
  for (int pp = 0; pp < C::PPG; ++pp) {
    const uint32_t o = ob + (uint32_t)(((p_lo + pp) * 16 + 4 * g) * 2);
    const u32x2 v = {pack_bf16(acc[pp][0], acc[pp][1]), pack_bf16(acc[pp][2], acc[pp][3])};
    __builtin_amdgcn_raw_buffer_store_b64(v, ry, (int)o, 0, 0);
  }
}

// One output unit: y_t = exp(cs_t) C~_t^T G + the intra-chunk term.
template <class C>
__device__ __forceinline__ void tok_output_unit(const TBuf& t, const rsrc& ry, uint32_t rowX,
                                                int qb, int p_lo) {
  constexpr int R = C::R, PPG = C::PPG;
  const int li = threadIdx.x & 15;
  const uint32_t qrow = (uint32_t)(qb * 16 + li);
  f32x4 acc[PPG];
#pragma unroll
  for (int pp = 0; pp < PPG; ++pp) acc[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
  tok_inter<C>(t.G, t.C, qrow, p_lo, __expf(t.sc[(qb * 16 + li) / R]), acc);
  tok_intra<C>(t, qb, p_lo, acc);
  tok_unit_store<C>(ry, rowX, qb, p_lo, acc);
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
__device__ __forceinline__ int tok_segment(const PrefillArgs& a, int ticket,
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
    const TDst d = {buf + C::oB, buf + C::oC, buf + C::oX, buf + C::oTh, buf + C::oRaw};
    if (i < K)
      tok_issue<C, false>(a, s, s.c0 + i, d);
    else
      tok_issue<C, true>(a, s, s.c0 + i - K, d);
  };

  f32x4 stt[kMaxStTiles];
#pragma unroll
  for (int q = 0; q < kMaxStTiles; ++q) stt[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  double sang = 0.0;  // lanes < NPW: the segment's angle of pair wave * NPW + lane
  float seg_logdecay = 0.f;
  int done_prev = 0;

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
      // no counter is touched after the chain: count the workgroup done
      // here, so the count's round trip overlaps the output pass
      done_prev = pf::finish_count(a);
    }
  }
  return done_prev;
}

template <class C>
__global__ void __launch_bounds__(kT) prefill_tok_kernel(PrefillArgs a_in) {
  extern __shared__ __align__(16) unsigned char smem[];
  PrefillArgs a = a_in;
  a.N = C::N;
  int* s_misc = reinterpret_cast<int*>(smem + C::oMisc);
  const int ticket = pf::take_ticket(a, s_misc);
  int done_prev;
  if (ticket >= 0 && ticket < (int)gridDim.x) {
    done_prev = tok_segment<C>(a, ticket, smem);
  } else {
    pf::bad_ticket(a);
    done_prev = pf::finish_count(a);
  }
  pf::finish_reset(a, done_prev, s_misc);
}

template <class C>
hipError_t launch_tok(const PrefillArgs& a, hipStream_t stream) {
  const hipError_t attr = lds_limit(reinterpret_cast<const void*>(&prefill_tok_kernel<C>), C::kTotal);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((prefill_tok_kernel<C>), dim3(a.nb * a.H * a.nSeg), dim3(kT), C::kTotal,
                     stream, a);
  return hipGetLastError();
}

// Output unit of the single pass (rank 1, query block qb, PPG p-tiles from
// p_lo):
//   y_t = exp(cs_t) C~_t^T G + sum_u W[t,u] (C~_t^T B~_u) x_u^T.
// The query fragments are read once for the inter-chunk term and every pair
// of key blocks, and each pair requests all its LDS operands (key
// fragments, key scalars, x fragments) before its first product: the mask's
// exponentials are kept out of a branch by an empty asm statement, which
// the scheduler does not move loads across.
template <class C>
__device__ __forceinline__ void tok1_unit(const TBuf& t, int qb, int p_lo, int kb0,
                                          f32x4 (&acc)[C::PPG]) {
  using M = typename C::M;
  constexpr int PPG = C::PPG, NK = C::N / M::K;
  static_assert(C::R == 1, "rank 1");
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const uint32_t qrow = (uint32_t)(qb * 16 + li);
  const int tq = qb * 16 + li;
  bf16x8 fq[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) fq[k] = frag_row(t.C, qrow, k * M::K);
  const float csq = t.cs[tq];
  {
    f32x4 gi[PPG];
#pragma unroll
    for (int pp = 0; pp < PPG; ++pp) gi[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
      for (int pp = 0; pp < PPG; ++pp)
        gi[pp] = M::mma(frag_row(t.G, (uint32_t)((p_lo + pp) * 16 + li), k * M::K), fq[k], gi[pp]);
    const float eq = __expf(csq);
#pragma unroll
    for (int pp = 0; pp < PPG; ++pp)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[pp][j] = gi[pp][j] * eq;
  }
  for (int kb = kb0; kb <= qb; kb += 2) {
    bf16x8 fk[2][NK], fx[PPG];
    float4 c4[2], ga4[2], go4[2];
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
      for (int i = 0; i < 2; ++i) fk[i][k] = frag_row(t.B, (uint32_t)((kb + i) * 16 + li), k * M::K);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row0 = (kb + i) * 16 + 4 * g;
      c4[i] = *reinterpret_cast<const float4*>(t.cs + row0);
      ga4[i] = *reinterpret_cast<const float4*>(t.gs + row0);
      go4[i] = *reinterpret_cast<const float4*>(t.gs + kL + row0);
    }
    // x^T with the scores' slot order: keys 16 kb + 4g .. + 3, then + 16
    const uint32_t r0 = (uint32_t)(kb * 16 + 4 * g), r1 = r0 + 16;
#pragma unroll
    for (int pp = 0; pp < PPG; ++pp) fx[pp] = frag_tr(t.X, r0, r1, p_lo + pp);
    f32x4 sct[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
      for (int i = 0; i < 2; ++i) sct[i] = M::mma(fk[i][k], fq[k], sct[i]);
    float kcs[2][4], kga[2][4], kgom[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      kcs[i][0] = c4[i].x; kcs[i][1] = c4[i].y; kcs[i][2] = c4[i].z; kcs[i][3] = c4[i].w;
      kga[i][0] = ga4[i].x; kga[i][1] = ga4[i].y; kga[i][2] = ga4[i].z; kga[i][3] = ga4[i].w;
      kgom[i][0] = go4[i].x; kgom[i][1] = go4[i].y; kgom[i][2] = go4[i].z; kgom[i][3] = go4[i].w;
    }
    pf::mask_scores<1, 2>(sct, kcs, kga, kgom, kb, g, tq, csq);
    bf16x8 fs;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      fs[j] = from_f32<bf16>(sct[0][j]);
      fs[4 + j] = from_f32<bf16>(sct[1][j]);
    }
#pragma unroll
    for (int pp = 0; pp < PPG; ++pp) acc[pp] = M::mma(fx[pp], fs, acc[pp]);
  }
}

// Hand-over of masked scores inside a step of the single pass.  The waves
// of query blocks 2 and 3 have two pairs of key blocks, the others one; so
// the waves of blocks 0 and 1 first compute the masked scores of query
// blocks 2 and 3 against key blocks 0 and 1 (one 16 x 16 block each, in the
// accumulator layout the product with x takes as its operand) and leave
// them in `ex` (2 KB of LDS) with a workgroup-scope release count; the
// others take them once the count shows all four, with an acquire load.
// Lane (g, c) of block kb holds keys 16 kb + 4g .. + 3 of query column c.
template <class C>
__device__ __forceinline__ void tok1_scores_give(const TBuf& t, uint32_t* ex, int* flag) {
  using M = typename C::M;
  constexpr int NK = C::N / M::K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int qx = 2 + wave / 2, kb = wave % 2;
  const int tq = qx * 16 + li;
  bf16x8 fk[NK], fq[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    fk[k] = frag_row(t.B, (uint32_t)(kb * 16 + li), k * M::K);
    fq[k] = frag_row(t.C, (uint32_t)tq, k * M::K);
  }
  const int row0 = kb * 16 + 4 * g;
  const float4 c4 = *reinterpret_cast<const float4*>(t.cs + row0);
  const float4 ga4 = *reinterpret_cast<const float4*>(t.gs + row0);
  const float4 go4 = *reinterpret_cast<const float4*>(t.gs + kL + row0);
  const float csq = t.cs[tq];
  f32x4 sct[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int k = 0; k < NK; ++k) sct[0] = M::mma(fk[k], fq[k], sct[0]);
  const float kcs[1][4] = {{c4.x, c4.y, c4.z, c4.w}};
  const float kga[1][4] = {{ga4.x, ga4.y, ga4.z, ga4.w}};
  const float kgom[1][4] = {{go4.x, go4.y, go4.z, go4.w}};
  pf::mask_scores<1, 1>(sct, kcs, kga, kgom, kb, g, tq, csq);
  reinterpret_cast<u32x2*>(ex)[(qx - 2) * 128 + kb * 64 + lane] =
      u32x2{pack_bf16(sct[0][0], sct[0][1]), pack_bf16(sct[0][2], sct[0][3])};
  // one count per wave (the release waits for all of the wave's stores)
  if (lane == 0) __hip_atomic_fetch_add(flag, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The other side: y += (masked scores of key blocks 0 and 1) x, for query
// block qb (2 or 3) and this wave's p-tiles, once the count reaches
// `target`.  The wait is bounded (the givers are waves of this workgroup
// with no wait of their own before they give); one that ran out would set
// error word 1, as a timed-out chain wait does.
template <class C>
__device__ __forceinline__ void tok1_scores_take(const PrefillArgs& a, const TBuf& t,
                                                 const uint32_t* ex, int* flag, int target,
                                                 int qb, int p_lo, f32x4 (&acc)[C::PPG]) {
  using M = typename C::M;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  bf16x8 fx[C::PPG];
  const uint32_t r0 = (uint32_t)(4 * g), r1 = r0 + 16;
#pragma unroll
  for (int pp = 0; pp < C::PPG; ++pp) fx[pp] = frag_tr(t.X, r0, r1, p_lo + pp);
  int spins = 0;
  while (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > (1 << 20)) {
      // (cannot happen while the givers run; reported as a timed-out wait)
      __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
  }
  const u32x2 v0 = reinterpret_cast<const u32x2*>(ex)[(qb - 2) * 128 + lane];
  const u32x2 v1 = reinterpret_cast<const u32x2*>(ex)[(qb - 2) * 128 + 64 + lane];
  const bf16x8 fs = __builtin_bit_cast(bf16x8, u32x4{v0[0], v0[1], v1[0], v1[1]});
#pragma unroll
  for (int pp = 0; pp < C::PPG; ++pp) acc[pp] = M::mma(fx[pp], fs, acc[pp]);
}

// ---- single pass -----------------------------------------------------------
// A segment of K <= kK1 chunks in one walk over its inputs.  Each step
// stages, rotates and multiplies one chunk as the output pass does, but
// from the segment's zero-entry state G_c (the local pass's state): its
// outputs are complete except for the entry state's share, and the same
// step advances G_c.  Rotated C~, the per-token scalars and the chunk's
// rotation stay in the LDS and the partial outputs in the wave's registers
// until the chain has given the true entry state h_in.  Since the state is
// linear in its entry, a chunk's true state is G_c + E_c with E_0 = h_in
// and E_{c+1} = R(Phi_c) exp(l_c) E_c, so the correction is
//   y_t += exp(cs_t) C~_t^T E_c,
// one 64 x 64 x 64 product per chunk: no input is read twice and no token
// rotated twice.  A sequence's first segment (entry zero) writes y as it
// goes and has no correction.
// The chain's view of a configuration with fewer aggregates in flight.
template <class C>
struct TChain : C {
  static constexpr int kAggBatch = 2;
};

// The single pass keeps the state in the first kNsw1 waves (4 tiles each):
// they are the waves of query blocks 0 and 1, whose output units are the
// shorter (one pair of key blocks against two), so the state update and its
// LDS copy run while the other waves still multiply.
constexpr int kNsw1 = 4;

template <class C>
__device__ __forceinline__ void tok1_correct_state(f32x4 (&e)[kMaxStTiles], const float* ang,
                                                   float d) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int nt = wave % C::NNT;
  const float2 f = *reinterpret_cast<const float2*>(ang + nt * 8 + 2 * g);
  const float2 q0 = make_float2(__builtin_amdgcn_cosf(f.x), __builtin_amdgcn_sinf(f.x));
  const float2 q1 = make_float2(__builtin_amdgcn_cosf(f.y), __builtin_amdgcn_sinf(f.y));
#pragma unroll
  for (int m = 0; m < C::NTILES / kNsw1; ++m) {
    const float v0 = d * e[m][0], v1 = d * e[m][1];
    const float v2 = d * e[m][2], v3 = d * e[m][3];
    e[m][0] = q0.x * v0 - q0.y * v1;
    e[m][1] = q0.y * v0 + q0.x * v1;
    e[m][2] = q1.x * v2 - q1.y * v3;
    e[m][3] = q1.y * v2 + q1.x * v3;
  }
}

// This wave's state tiles (tile i = wave + kNsw1 m: n-tile i % NNT, p-tile
// i / NNT; lane (g, c) holds rows 4g..4g+3 of column c) into the tile [P][N]
// (bf16).
template <class C>
__device__ __forceinline__ void tok1_state_to_lds(const f32x4 (&stt)[kMaxStTiles], const Tile& tG) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  if (wave >= kNsw1) return;
#pragma unroll
  for (int m = 0; m < C::NTILES / kNsw1; ++m) {
    const int i = wave + kNsw1 * m;
    const int nt = i % C::NNT, pt = i / C::NNT;
    tG.ref<u32x2>((uint32_t)(pt * 16 + li), (uint32_t)((nt * 16 + 4 * g) * 2)) =
        u32x2{pack_bf16(stt[m][0], stt[m][1]), pack_bf16(stt[m][2], stt[m][3])};
  }
}

// Chunk state folded into the state waves' tiles: stt <- R(Phi_c)(d stt +
// S), S = sum over tokens of w_u B~_u x_u^T, the A operand B~ with each
// token's slot scaled by its state weight (t.gs), the rotation from the
// chunk's angles (t.ang).
template <class C>
__device__ __forceinline__ void tok1_state_update(const TBuf& t, float d,
                                                  f32x4 (&stt)[kMaxStTiles]) {
  using M = typename C::M;
  constexpr int TPW = C::NTILES / kNsw1;
  static_assert(TPW <= kMaxStTiles && kNsw1 % C::NNT == 0, "state tiles of a wave share an n-tile");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  if (wave >= kNsw1) return;
  const int nt = wave % C::NNT;
  // the decayed state is the accumulator the chunk's products add to
#pragma unroll
  for (int m = 0; m < TPW; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) stt[m][j] *= d;
#pragma unroll
  for (int k0 = 0; k0 < C::LR; k0 += M::K) {
    // slots 0..7 are tokens r0 .. r0 + 7
    const uint32_t r0 = (uint32_t)(k0 + 8 * g);
    bf16x8 fa = frag_tr(t.B, r0, r0 + 4, nt);
    const float4 w0 = *reinterpret_cast<const float4*>(t.gs + 2 * kL + r0);
    const float4 w1 = *reinterpret_cast<const float4*>(t.gs + 2 * kL + r0 + 4);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) fa[j] = from_f32<bf16>(to_f32(fa[j]) * wv[j]);
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int pt = (wave + kNsw1 * m) / C::NNT;
      stt[m] = M::mma(fa, frag_tr(t.X, r0, r0 + 4, pt), stt[m]);
    }
  }
  // rows 4g .. 4g + 3 of n-tile nt: pairs 8 nt + 2g and 8 nt + 2g + 1
  const float2 f = *reinterpret_cast<const float2*>(t.ang + nt * 8 + 2 * g);
  const float2 q0 = make_float2(__builtin_amdgcn_cosf(f.x), __builtin_amdgcn_sinf(f.x));
  const float2 q1 = make_float2(__builtin_amdgcn_cosf(f.y), __builtin_amdgcn_sinf(f.y));
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const float v0 = stt[m][0], v1 = stt[m][1], v2 = stt[m][2], v3 = stt[m][3];
    stt[m][0] = q0.x * v0 - q0.y * v1;
    stt[m][1] = q0.y * v0 + q0.x * v1;
    stt[m][2] = q1.x * v2 - q1.y * v3;
    stt[m][3] = q1.y * v2 + q1.x * v3;
  }
}

// The uniform values of the segment of a ticket.
template <class C>
__device__ __forceinline__ TCtx tok_ctx(const PrefillArgs& a, int ticket) {
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
  s.Ah = 0.f;
  return s;
}

// Staging of the single pass: chunk i of the segment into ring buffer i % 3
// (B, x, theta, dt and lam) and C slot i.  (The offsets are made opaque so
// that per-lane addresses are formed at each use rather than kept live
// across the loop.)
template <class C>
__device__ __forceinline__ void tok1_issue(const PrefillArgs& a, const TCtx& s, int i,
                                           unsigned char* smem) {
  if (i >= s.c1 - s.c0) return;
  unsigned char* r = smem + pf::opaque_u((uint32_t)(i % 3) * C::k1Ring);
  unsigned char* pc = smem + pf::opaque_u(C::o1Per + (uint32_t)i * C::k1Per);
  const TDst d = {r + C::o1B, pc + C::o1C, r + C::o1X, r + C::o1Th, r + C::o1Raw};
  tok_issue<C, true, true>(a, s, s.c0 + i, d);
}

// One segment in one pass.  Counts the workgroup done once the chain is
// over (pf::finish_count) and returns that count (thread 0), so that its
// round trip overlaps the correction.
template <class C>
__device__ __forceinline__ int tok1_segment(const PrefillArgs& a, int ticket,
                                            unsigned char* smem) {
  constexpr int KK = C::kK1, PPG = C::PPG;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15;
  TCtx s = tok_ctx<C>(a, ticket);
  s.Ah = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.A[s.h])));
  const bool has_lam = a.lam != nullptr;
  // the sequence's first segment starts from zero: its outputs are final
  const bool direct = s.seg == 0 && !a.cont;
  int* s_misc = reinterpret_cast<int*>(smem + C::o1Misc);
  float2* s_srot = reinterpret_cast<float2*>(smem + C::o1Srot);
  const int K = s.c1 - s.c0;  // 1 .. KK
  // this wave's output unit: query block qb, p-tiles p_lo .. p_lo + PPG - 1
  const int qb = wave / C::NPG, p_lo = (wave % C::NPG) * PPG;
  const uint32_t qrow = (uint32_t)(qb * 16 + li);
  const int tq = qb * 16 + li;

  auto ring = [&](int i) { return smem + pf::opaque_u((uint32_t)(i % 3) * C::k1Ring); };
  auto dbl = [&](int i) {
    return smem + pf::opaque_u(C::o1Dbl + (uint32_t)(i & 1) * C::k1Dbl);
  };
  auto per = [&](int i) { return smem + pf::opaque_u(C::o1Per + (uint32_t)i * C::k1Per); };
  auto issue = [&](int i) { tok1_issue<C>(a, s, i, smem); };
  auto yrange = [&](int i) {
    const int t0 = (s.c0 + i) * kL;
    const int len = min(kL, a.T - t0);
    const size_t hrow = ((size_t)s.b * a.T + t0) * a.H + s.h;
    constexpr uint32_t yb = C::R * C::P * 2;
    return make_rsrc(static_cast<unsigned char*>(a.y) + hrow * yb,
                     (uint32_t)(len - 1) * s.rowX + yb);
  };

  f32x4 stt[kMaxStTiles];
#pragma unroll
  for (int q = 0; q < kMaxStTiles; ++q) stt[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  // partial outputs and chunk decays of the segment's chunks, oldest first
  // (a queue shifted each step, so every index is static)
  f32x4 yp[KK][PPG];
  float dec[KK];
#pragma unroll
  for (int c = 0; c < KK; ++c) {
    dec[c] = 0.f;
#pragma unroll
    for (int pp = 0; pp < PPG; ++pp) yp[c][pp] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  double sang = 0.0;  // lanes < NPW: the segment's angle of pair wave * NPW + lane
  float seg_logdecay = 0.f;

  if (tid == 0) s_misc[8] = 0;  // the scores hand-over count
  issue(0);
  __builtin_amdgcn_s_waitcnt(0);
  issue(1);
  __syncthreads();

  for (int i = 0; i < K; ++i) {
    unsigned char* r = ring(i);
    unsigned char* d2 = dbl(i);
    unsigned char* pc = per(i);
    TBuf t;
    t.base = r;
    t.B = tile_at(r + C::o1B, C::kRowN);
    t.C = tile_at(pc + C::o1C, C::kRowN);
    t.W = t.B;  // (no weighted tile in the single pass)
    t.X = tile_at(r + C::o1X, C::kRowP);
    t.Th = tile_at(r + C::o1Th, C::kRowTh);
    t.G = tile_at(d2 + C::o1G, C::kRowN);
    t.raw = reinterpret_cast<float*>(r + C::o1Raw);
    t.sc = nullptr;
    t.rot = nullptr;
    t.cs = reinterpret_cast<float*>(pc + C::o1Cs);
    t.gs = reinterpret_cast<float*>(d2 + C::o1Gs);
    t.ang = reinterpret_cast<float*>(pc + C::o1Ang);
    const float cse = tok_rotate<C, true, true>(t, has_lam, s.Ah, sang);
    // (zero in the first step: one code path for every step)
    tok1_state_to_lds<C>(stt, t.G);
    // the next chunk's loads (issued a step ago) have landed
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x4 acc[PPG];
    {
      // the scores hand-over lives in this chunk's theta area (read only by
      // the rotation before the barrier, reloaded two steps later)
      uint32_t* ex = reinterpret_cast<uint32_t*>(r + C::o1Th);
      int* flag = s_misc + 8;
      if (wave < 4) {
        tok1_scores_give<C>(t, ex, flag);
        tok1_unit<C>(t, qb, p_lo, 0, acc);
      } else {
        tok1_unit<C>(t, qb, p_lo, 2, acc);
        tok1_scores_take<C>(a, t, ex, flag, 4 * (i + 1), qb, p_lo, acc);
      }
    }
    if (direct) {
      tok_unit_store<C>(yrange(i), s.rowX, qb, p_lo, acc);
    } else {
#pragma unroll
      for (int c = 0; c + 1 < KK; ++c)
#pragma unroll
        for (int pp = 0; pp < PPG; ++pp) yp[c][pp] = yp[c + 1][pp];
#pragma unroll
      for (int pp = 0; pp < PPG; ++pp) yp[KK - 1][pp] = acc[pp];
    }
    const float d = __expf(cse);
    tok1_state_update<C>(t, d, stt);
#pragma unroll
    for (int c = 0; c + 1 < KK; ++c) dec[c] = dec[c + 1];
    dec[KK - 1] = d;
    // the ring buffer of chunk i + 2 was last read in the previous step's
    // MFMA phase, which every wave finished before this step's barrier
    issue(i + 2);
    seg_logdecay += cse;
  }
  // chunk c's partial outputs and decay to index c
  for (int j = K; j < KK; ++j) {
#pragma unroll
    for (int c = 0; c + 1 < KK; ++c) {
      dec[c] = dec[c + 1];
#pragma unroll
      for (int pp = 0; pp < PPG; ++pp) yp[c][pp] = yp[c + 1][pp];
    }
  }

  // ---- the chain (chain_phase): the true entry state ------------------------
  if (lane < C::NPW) {
    const float f = static_cast<float>(sang);
    s_srot[wave * C::NPW + lane] = make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
  }
  __syncthreads();  // s_srot; every MFMA read of the last step is done
  const WaveRoles wr = {0, 0, 0, 0, kNsw1};
  f32x4 ent[kMaxStTiles];
  // (the state waves hold four tiles each beside the partial outputs: two
  // aggregates in flight at a time)
  pf::chain_phase<TChain<C>>(a, wr, s.seg, s.bh, ticket, __expf(seg_logdecay), s_srot, s_misc, stt,
                          ent);
  __builtin_amdgcn_s_waitcnt(0);
  // no counter is touched after the chain
  const int done_prev = pf::finish_count(a);
  if (direct) return done_prev;

  // ---- correction: y_t += exp(cs_t) C~_t^T E_c ------------------------------
  // E_c as [P][N] bf16 tiles in the ring (free now: the chain's barriers
  // follow the last step's reads)
#pragma unroll
  for (int c = 0; c < KK; ++c) {
    if (c < K) {
      tok1_state_to_lds<C>(ent, tile_at(smem + (uint32_t)c * (C::P * C::kRowN), C::kRowN));
      if (c + 1 < K && wave < kNsw1)
        tok1_correct_state<C>(ent, reinterpret_cast<const float*>(per(c) + C::o1Ang), dec[c]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < KK; ++c) {
    if (c < K) {
      unsigned char* pc = per(c);
      const float* cs = reinterpret_cast<const float*>(pc + C::o1Cs);
      tok_inter<C>(tile_at(smem + (uint32_t)c * (C::P * C::kRowN), C::kRowN),
                   tile_at(pc + C::o1C, C::kRowN), qrow, p_lo, __expf(cs[tq]), yp[c]);
      tok_unit_store<C>(yrange(c), s.rowX, qb, p_lo, yp[c]);
    }
  }
  return done_prev;
}

template <class C>
__global__ void __launch_bounds__(kT) prefill_tok1_kernel(PrefillArgs a_in) {
  extern __shared__ __align__(16) unsigned char smem[];
  PrefillArgs a = a_in;
  a.N = C::N;
  int* s_misc = reinterpret_cast<int*>(smem + C::o1Misc);
  const int ticket = pf::take_ticket(a, s_misc);
  int done_prev;
  if (ticket >= 0 && ticket < (int)gridDim.x) {
    done_prev = tok1_segment<C>(a, ticket, smem);
  } else {
    pf::bad_ticket(a);
    done_prev = pf::finish_count(a);
  }
  pf::finish_reset(a, done_prev, s_misc);
}

template <class C>
hipError_t launch_tok1(const PrefillArgs& a, hipStream_t stream) {
  const hipError_t attr =
      lds_limit(reinterpret_cast<const void*>(&prefill_tok1_kernel<C>), C::k1Total);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((prefill_tok1_kernel<C>), dim3(a.nb * a.H * a.nSeg), dim3(kT), C::k1Total,
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
  // segments of up to kK1 chunks take the single pass, longer ones the two
  // passes (the segment rule gives 8 chunks at the SISO bench shape)
  using C1 = TCfg<1, 64, 64>;
  static_assert(C1::k1Fits, "the single pass fits the LDS at N = P = 64");
  if (a.K <= C1::kK1) {
    *taken = true;
    return launch_tok1<C1>(a, stream);
  }
  return try_tok<1, 64, 64>(a, stream, taken);
}

}  // namespace pt
}  // namespace m3
