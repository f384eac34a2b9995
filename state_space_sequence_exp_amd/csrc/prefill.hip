// prefill.hip -- chunked prefill of the Mamba-3 recurrence on gfx950, as one
// fused kernel that reads every input from HBM once.
//
// The sequence of each (batch b, head h) is cut into chunks of L tokens and
// the chunks into segments of K chunks.  One workgroup (512 threads) owns one
// segment and runs three phases:
//
//  1. Local pass.  For each chunk: per-token log-decay prefix sums cs_u (wave
//     scan), trapezoid weights gamma_u = lam_u dt_u and omega_u = (1 -
//     lam_{u+1}) dt_{u+1}, chunk-local cumulative angles phi_u[k] (segmented
//     scan per rotation pair), rotated inputs B~_u = R(phi_u)^T B_u (the
//     data-dependent RoPE of Proposition 3, Mamba-3 paper summary), the chunk
//     state S_c = sum_u exp(cs_e - cs_u)(gamma_u + omega_u) B~_u x_u^T on
//     MFMA, and the chunk-level recurrence G <- R(Phi_c)(exp(cs_e) G + S_c)
//     from G = 0.  The result is the segment's exit state for a zero entry
//     state, plus the segment's total decay and total angle.
//  2. Chain.  Wait for the exit state of the previous segment of the same
//     sequence, combine (the recurrence is linear: E_exit = R(Phi)(D E_entry)
//     + E_local), publish this segment's exit state.
//  3. Output pass.  Walk the chunks again from the true entry state:
//         y_t = exp(cs_t) C~_t^T G_c
//             + sum_{u<=t} exp(cs_t - cs_u)(gamma_u + [u<t] omega_u)(C~_t^T B~_u) x_u^T
//     i.e. the chunk's structured mask (decay matrix x 2-band trapezoid
//     matrix; Mamba-3 paper translation, section 3.1, equation 7) applied to
//     C~ B~^T on MFMA, plus the inter-chunk term, then the same chunk-level
//     recurrence to the next chunk.  Its inputs were read moments earlier by
//     phase 1, so the re-read is served by the caches, not HBM.
//
// Frames.  Angles restart at every chunk, so the entry state G_c of a chunk
// is in the unrotated (API) frame, and the previous token's trapezoid term
// omega B x^T is folded into it: G_c = h_{cL-1} + omega_{cL-1} B_{cL-1}
// x_{cL-1}^T.  No halo token is needed inside a chunk and every angle stays
// bounded by one chunk's sum.  Chunk and segment angle totals are summed in
// double and take the accurate sine/cosine, since the chain multiplies their
// rotations over the whole sequence.
//
// Work order and the chain.  Workgroups take tickets from a counter; ticket
// t is segment t / (B*H) of sequence t % (B*H).  A workgroup only waits for a
// smaller ticket, which is held by a running workgroup, so the grid always
// drains.  Exit states travel through a two-slot ring per sequence with
// device-coherent (sc1) stores and loads, and a per-sequence counter that is
// raised only after the stores have completed; the wait is bounded and
// raises an error word instead of hanging.
//
// Register and LDS layout.  Both MFMA operands keep their contraction
// dimension contiguous in LDS wherever possible: C~, B~ as [row][N], X^T as
// [p][row], the state copy as [P][N]; the chunk-state contraction reads B~
// transposed.  The state itself lives in MFMA accumulator layout ([N][P]
// tiles, rows n = 4g..4g+3 in one lane), so a rotation pair (2k, 2k+1) is
// always inside one lane.  Each thread stages the next chunk's raw inputs in
// registers while the current chunk computes.  R, P, the storage type and the
// staging depth are compile-time, so index arithmetic is shifts and masks.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

constexpr int kW = kThreads / kWave;  // waves per workgroup
constexpr int kSpinLimit = 1 << 18;   // bounded wait (a few hundred ms)

template <typename T_, int R_, int P_, int MV_>
struct Cfg {
  using T = T_;
  static constexpr int R = R_;    // MIMO rank
  static constexpr int P = P_;    // head dimension
  static constexpr int MV = MV_;  // staged 16-byte vectors per thread per tile
  static constexpr int es = sizeof(T_);
  static constexpr int vec = 16 / es;  // elements per 16-byte vector
  // C is staged a chunk ahead with the other inputs when the staging is
  // small; with four vectors per tile it would not fit the register budget
  // next to the compute, so it is loaded when its chunk is committed.
  static constexpr bool kStageC = MV_ <= 2;
};

struct Seq {
  int b, h, bh, seg, c0, c1;
};

// The 16-byte vectors of a [rows][vpr] tile this thread moves:
// row = row0 + i * rpp, column col (vpr divides kThreads).
struct VecMap {
  int row0, col, rpp;
};
__device__ __forceinline__ VecMap vec_map(int vpr) {
  const int tid = threadIdx.x;
  return VecMap{tid / vpr, tid % vpr, kThreads / vpr};
}

struct Maps {
  VecMap bn;  // B and C rows (N elements)
  VecMap xp;  // x rows (P elements)
  VecMap th;  // theta rows (N/2 floats)
};

template <class C>
struct Stage {
  u32x4 bv[C::MV], cv[C::kStageC ? C::MV : 1], xv[C::MV], tv[C::MV];
  float dtv, lamv;
};

// Element q of a 16-byte vector of T (q is a compile-time constant after
// unrolling, so this folds to register moves).
template <typename T>
__device__ __forceinline__ T vec_elem(const u32x4& v, int q);
template <>
__device__ __forceinline__ float vec_elem<float>(const u32x4& v, int q) {
  return __uint_as_float(v[q]);
}
template <>
__device__ __forceinline__ bf16 vec_elem<bf16>(const u32x4& v, int q) {
  const unsigned w = v[q >> 1];
  const unsigned short h = (q & 1) ? (unsigned short)(w >> 16) : (unsigned short)(w & 0xffffu);
  return __builtin_bit_cast(bf16, h);
}

// Global -> registers for chunk c (c < nC).  The loads carry no condition:
// rows past the chunk or the sequence are clamped to an in-range address and
// masked at commit time, so the compiler has no reason to wait for them
// before the data is used.
template <class C, bool kWithC>
__device__ __forceinline__ void issue_loads(const PrefillArgs& a, const Seq& s, const Maps& mp,
                                           int c, Stage<C>& st) {
  constexpr int R = C::R;
  const int t0 = c * a.L;
  const int len = min(a.L, a.T - t0);
  const int LR = a.L * R;
  const size_t tokrow = (size_t)a.H * R;  // rows per token across heads
  const size_t base_row = ((size_t)s.b * a.T + t0) * tokrow + (size_t)s.h * R;
  const unsigned char* Bg = static_cast<const unsigned char*>(a.B);
  const unsigned char* Cg = static_cast<const unsigned char*>(a.C);
  const unsigned char* Xg = static_cast<const unsigned char*>(a.x);
#pragma unroll
  for (int i = 0; i < C::MV; ++i) {
    const int row = min(mp.bn.row0 + i * mp.bn.rpp, LR - 1);
    const int u = min(row / R, len - 1);
    const size_t off = (base_row + (size_t)u * tokrow + row % R) * a.N * C::es + mp.bn.col * 16;
    st.bv[i] = *reinterpret_cast<const u32x4*>(Bg + off);
    if constexpr (kWithC && C::kStageC) st.cv[i] = *reinterpret_cast<const u32x4*>(Cg + off);
  }
#pragma unroll
  for (int i = 0; i < C::MV; ++i) {
    const int row = min(mp.xp.row0 + i * mp.xp.rpp, LR - 1);
    const int u = min(row / R, len - 1);
    st.xv[i] = *reinterpret_cast<const u32x4*>(
        Xg + (base_row + (size_t)u * tokrow + row % R) * C::P * C::es + mp.xp.col * 16);
  }
  const int npair = a.N / 2;
  const size_t throw_ = ((size_t)s.b * a.T + t0) * a.H + s.h;  // [B,T,H] row of token t0
#pragma unroll
  for (int i = 0; i < C::MV; ++i) {
    const int u = min(min(mp.th.row0 + i * mp.th.rpp, a.L - 1), len - 1);
    st.tv[i] = *reinterpret_cast<const u32x4*>(a.theta + (throw_ + (size_t)u * a.H) * npair +
                                               mp.th.col * 4);
  }
  // dt and lam of tokens t0 .. t0 + L (the extra one feeds omega)
  const int tt = min(t0 + min((int)threadIdx.x, a.L), a.T - 1);
  const size_t i = ((size_t)s.b * a.T + tt) * a.H + s.h;
  st.dtv = a.dt[i];
  st.lamv = a.lam[i];
}

// Registers -> LDS for chunk c: raw B (and C) rows, X^T, theta, dt/lam, with
// rows past the end of the sequence zeroed.
template <class C, bool kWithC>
__device__ __forceinline__ void commit_stage(const PrefillArgs& a, const Seq& s, const Maps& mp,
                                             const ChunkLayout& lay, int c, const Stage<C>& st,
                                             unsigned char* smem) {
  using T = typename C::T;
  constexpr int R = C::R, vec = C::vec;
  const int tid = threadIdx.x;
  const int LR = lay.LR;
  const int t0 = c * a.L;
  const int len = min(a.L, a.T - t0);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  T* sB = reinterpret_cast<T*>(smem + lay.off_B);
  T* sC = reinterpret_cast<T*>(smem + lay.off_C);
  T* sXT = reinterpret_cast<T*>(smem + lay.off_XT);
  if constexpr (kWithC && !C::kStageC) {
    // C now, straight from global memory
    const size_t tokrow = (size_t)a.H * R;
    const size_t base_row = ((size_t)s.b * a.T + t0) * tokrow + (size_t)s.h * R;
    const unsigned char* Cg = static_cast<const unsigned char*>(a.C);
    u32x4 cv[C::MV];
#pragma unroll
    for (int i = 0; i < C::MV; ++i) {
      const int row = min(mp.bn.row0 + i * mp.bn.rpp, LR - 1);
      const int u = min(row / R, len - 1);
      cv[i] = *reinterpret_cast<const u32x4*>(
          Cg + (base_row + (size_t)u * tokrow + row % R) * a.N * C::es + mp.bn.col * 16);
    }
#pragma unroll
    for (int i = 0; i < C::MV; ++i) {
      const int row = mp.bn.row0 + i * mp.bn.rpp;
      if (row < LR)
        *reinterpret_cast<u32x4*>(sC + row * lay.ldN + mp.bn.col * vec) =
            row / R < len ? cv[i] : zero;
    }
  }
#pragma unroll
  for (int i = 0; i < C::MV; ++i) {
    const int row = mp.bn.row0 + i * mp.bn.rpp;
    if (row < LR) {
      const bool ok = row / R < len;
      *reinterpret_cast<u32x4*>(sB + row * lay.ldN + mp.bn.col * vec) = ok ? st.bv[i] : zero;
      if constexpr (kWithC && C::kStageC)
        *reinterpret_cast<u32x4*>(sC + row * lay.ldN + mp.bn.col * vec) = ok ? st.cv[i] : zero;
    }
  }
  // zero rows [LR, LRpad) of B (and C)
  const int vprN = a.N / vec;
  for (int i = tid; i < (lay.LRpad - LR) * vprN; i += kThreads) {
    const int row = LR + i / vprN, col = i % vprN;
    *reinterpret_cast<u32x4*>(sB + row * lay.ldN + col * vec) = zero;
    if constexpr (kWithC) *reinterpret_cast<u32x4*>(sC + row * lay.ldN + col * vec) = zero;
  }
#pragma unroll
  for (int i = 0; i < C::MV; ++i) {
    const int row = mp.xp.row0 + i * mp.xp.rpp;
    if (row < LR) {
      const u32x4 xv = row / R < len ? st.xv[i] : zero;
      T* dst = sXT + (mp.xp.col * vec) * lay.ldK + row;
#pragma unroll
      for (int q = 0; q < vec; ++q) dst[q * lay.ldK] = vec_elem<T>(xv, q);
    }
  }
  for (int i = tid; i < (lay.LRpad - LR) * C::P; i += kThreads) {
    const int col = LR + i % (lay.LRpad - LR), p = i / (lay.LRpad - LR);
    sXT[p * lay.ldK + col] = from_f32<T>(0.f);
  }
  float* s_th = reinterpret_cast<float*>(smem + lay.off_th);
  const int npair = a.N / 2;
#pragma unroll
  for (int i = 0; i < C::MV; ++i) {
    const int u = mp.th.row0 + i * mp.th.rpp;
    if (u < a.L)
      *reinterpret_cast<u32x4*>(s_th + u * npair + mp.th.col * 4) = u < len ? st.tv[i] : zero;
  }
  float* s_dtr = reinterpret_cast<float*>(smem + lay.off_dtr);
  float* s_lamr = reinterpret_cast<float*>(smem + lay.off_lamr);
  if (tid <= a.L) {
    const bool ok = t0 + tid < a.T;
    s_dtr[tid] = ok ? st.dtv : 0.f;
    s_lamr[tid] = ok ? st.lamv : 0.f;
  }
}

// Per-token scalars from the staged dt/lam: cs (inclusive prefix of dt*A),
// gamma, omega, dt, and the state weight w.  Padding tokens get zeros.  Ends
// with a barrier.
__device__ __forceinline__ void chunk_scalars(const PrefillArgs& a, const ChunkLayout& lay,
                                              int len, int t0, float Ah, unsigned char* smem) {
  const int tid = threadIdx.x;
  const float* s_dtr = reinterpret_cast<const float*>(smem + lay.off_dtr);
  const float* s_lamr = reinterpret_cast<const float*>(smem + lay.off_lamr);
  float* s_cs = reinterpret_cast<float*>(smem + lay.off_cs);
  float* s_gam = reinterpret_cast<float*>(smem + lay.off_gam);
  float* s_om = reinterpret_cast<float*>(smem + lay.off_om);
  float* s_dt = reinterpret_cast<float*>(smem + lay.off_dt);
  float* s_w = reinterpret_cast<float*>(smem + lay.off_w);
  if (tid < 2 * kWave) {
    const int u = tid;
    float d = 0.f, la = 0.f, om = 0.f;
    if (u < len) {
      d = s_dtr[u];
      la = s_lamr[u];
      if (t0 + u + 1 < a.T) om = (1.f - s_lamr[u + 1]) * s_dtr[u + 1];
    }
    const float cs = wave_incl_scan(d * Ah);
    s_cs[u] = cs;
    s_gam[u] = la * d;
    s_om[u] = om;
    s_dt[u] = d;
  }
  __syncthreads();
  if (tid >= kWave && tid < 2 * kWave) s_cs[tid] += s_cs[kWave - 1];
  __syncthreads();
  // weight of token u in the chunk's state: exp(cs_end - cs_u) (gamma_u + omega_u);
  // zero past L so that whole-vector reads need no bounds check
  if (tid < kLMax) s_w[tid] = tid < a.L ? __expf(s_cs[a.L - 1] - s_cs[tid]) * (s_gam[tid] + s_om[tid]) : 0.f;
  __syncthreads();
}

// R(phi)^T applied in place to the rotation pair at p (two adjacent elements).
__device__ __forceinline__ void rotate_pair_T(bf16* p, float cn, float sn) {
  const bf16x2 v = *reinterpret_cast<const bf16x2*>(p);
  const float x = static_cast<float>(v.x), y = static_cast<float>(v.y);
  const bf16x2 o = {from_f32<bf16>(cn * x + sn * y), from_f32<bf16>(-sn * x + cn * y)};
  *reinterpret_cast<bf16x2*>(p) = o;
}
__device__ __forceinline__ void rotate_pair_T(float* p, float cn, float sn) {
  const float2 v = *reinterpret_cast<const float2*>(p);
  *reinterpret_cast<float2*>(p) = make_float2(cn * v.x + sn * v.y, -sn * v.x + cn * v.y);
}

// An angle in radians (a double sum of float angles) reduced to [-pi, pi].
__device__ __forceinline__ double reduce_angle(double a) {
  constexpr double kTwoPi = 6.283185307179586476925;
  return a - kTwoPi * __builtin_rint(a * (1.0 / kTwoPi));
}

// Chunk-local cumulative angles and rotated inputs, in place in LDS: B~
// (and C~) overwrite the raw rows; the chunk's total rotation goes to crot;
// with kAccumSeg the chunk's total angle is added to the segment sum.  Thread
// (pair kp, segment sg) scans tokens [sg*seglen, (sg+1)*seglen): the
// per-segment and per-chunk angle sums are accumulated in double (they feed
// the chain, which multiplies the rotations over the whole sequence); the
// running angle within the segment is a float reduced at every step.  Ends
// with a barrier.
template <class C, bool kWithC, bool kAccumSeg>
__device__ __forceinline__ void chunk_rotate(const PrefillArgs& a, const ChunkLayout& lay,
                                             int len, unsigned char* smem) {
  using T = typename C::T;
  constexpr int R = C::R;
  const int tid = threadIdx.x;
  const int npair = a.N / 2, nseg = kThreads / npair;
  const int kp = tid % npair, sg = tid / npair;
  const bool active = sg < nseg;
  const int seglen = (a.L + nseg - 1) / nseg;
  const int u0 = sg * seglen, u1 = min(a.L, u0 + seglen);
  const float* s_dt = reinterpret_cast<const float*>(smem + lay.off_dt);
  const float* s_th = reinterpret_cast<const float*>(smem + lay.off_th);
  double* s_part = reinterpret_cast<double*>(smem + lay.off_part);
  float2* s_crot = reinterpret_cast<float2*>(smem + lay.off_crot);
  double* s_sang = reinterpret_cast<double*>(smem + lay.off_sang);
  T* sB = reinterpret_cast<T*>(smem + lay.off_B);
  T* sC = reinterpret_cast<T*>(smem + lay.off_C);

  const int ulen = min(u1, len);
  double sum = 0.0;
  if (active)
    for (int u = u0; u < ulen; ++u) sum += static_cast<double>(s_dt[u] * s_th[u * npair + kp]);
  if (active) s_part[sg * npair + kp] = sum;
  __syncthreads();
  if (active) {
    double pre = 0.0;
    for (int q = 0; q < sg; ++q) pre += s_part[q * npair + kp];
    float phi = static_cast<float>(reduce_angle(pre));
    for (int u = u0; u < ulen; ++u) {
      phi = angle_add(phi, s_dt[u] * s_th[u * npair + kp]);
      float sn, cn;
      fast_sincos(phi, &sn, &cn);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        rotate_pair_T(sB + (u * R + r) * lay.ldN + 2 * kp, cn, sn);
        if constexpr (kWithC) rotate_pair_T(sC + (u * R + r) * lay.ldN + 2 * kp, cn, sn);
      }
    }
    if (u1 == a.L && u0 < a.L) {
      // the chunk's total angle; the chain multiplies its rotation over the
      // whole sequence, so it takes the accurate sine/cosine
      const double tot = pre + sum;
      float sn, cn;
      sincosf(static_cast<float>(reduce_angle(tot)), &sn, &cn);
      s_crot[kp] = make_float2(cn, sn);
      if constexpr (kAccumSeg) s_sang[kp] = reduce_angle(s_sang[kp] + tot);
    }
  }
  __syncthreads();
}

// Transposed fragment of B~ ([row][n] in LDS): lane holds column n and the
// K-slots k0 + g*KPL .. (rows of the chunk tile).
__device__ __forceinline__ bf16x8 load_frag_T(const bf16* sB, int ldN, int n, int k0) {
  const int g = (threadIdx.x & 63) >> 4;
  const bf16* p = sB + (k0 + g * 8) * ldN + n;
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = p[e * ldN];
  return f;
}
__device__ __forceinline__ float load_frag_T(const float* sB, int ldN, int n, int k0) {
  const int g = (threadIdx.x & 63) >> 4;
  return sB[(k0 + g) * ldN + n];
}

// The 8 token weights of chunk rows row0 .. row0+7 (row0 a multiple of 8);
// the weights are zero-padded past the chunk.
template <int R>
__device__ __forceinline__ void row_weights8(const float* s_w, int row0, float (&w)[8]) {
  if constexpr (R == 1) {
    const float4 a = *reinterpret_cast<const float4*>(s_w + row0);
    const float4 b = *reinterpret_cast<const float4*>(s_w + row0 + 4);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else if constexpr (R == 2) {
    const float4 a = *reinterpret_cast<const float4*>(s_w + row0 / 2);
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = e < 2 ? a.x : e < 4 ? a.y : e < 6 ? a.z : a.w;
  } else {
    const float2 a = *reinterpret_cast<const float2*>(s_w + row0 / 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = e < 4 ? a.x : a.y;
  }
}

// Fragment of X^T row p with every K-slot (a chunk row) scaled by its token's
// state weight (rows past LR are zero in X^T and have weight zero).
template <int R>
__device__ __forceinline__ bf16x8 load_frag_xw(const bf16* sXT, int ldK, int p, int k0,
                                               const float* s_w) {
  const int g = (threadIdx.x & 63) >> 4;
  const int row0 = k0 + g * 8;
  const bf16x8 x = *reinterpret_cast<const bf16x8*>(sXT + p * ldK + row0);
  float w[8];
  row_weights8<R>(s_w, row0, w);
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const bf16x2 h = {from_f32<bf16>(static_cast<float>(x[e]) * w[e]),
                      from_f32<bf16>(static_cast<float>(x[e + 1]) * w[e + 1])};
    f[e] = h.x;
    f[e + 1] = h.y;
  }
  return f;
}
template <int R>
__device__ __forceinline__ float load_frag_xw(const float* sXT, int ldK, int p, int k0,
                                              const float* s_w) {
  const int g = (threadIdx.x & 63) >> 4;
  const int row = k0 + g;
  return sXT[p * ldK + row] * s_w[row / R];
}

// Chunk state S_c = sum_u w_u B~_u x_u^T (MFMA) folded into the running state
// tiles: st <- R(Phi_c) (d st + S_c).  Tile m of this wave is i = wave + m*kW:
// n-tile i % (N/16), p-tile i / (N/16); lane holds rows n = 4g..4g+3.
template <class C>
__device__ __forceinline__ void state_update(const PrefillArgs& a, const ChunkLayout& lay,
                                             float d, f32x4 (&stt)[kMaxStTiles],
                                             const unsigned char* smem) {
  using T = typename C::T;
  using M = Mfma<T>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int ntn = a.N / 16, ntiles = ntn * (C::P / 16);
  const T* sB = reinterpret_cast<const T*>(smem + lay.off_B);
  const T* sXT = reinterpret_cast<const T*>(smem + lay.off_XT);
  const float* s_w = reinterpret_cast<const float*>(smem + lay.off_w);
  const float2* s_crot = reinterpret_cast<const float2*>(smem + lay.off_crot);
#pragma unroll
  for (int m = 0; m < kMaxStTiles; ++m) {
    const int i = wave + m * kW;
    if (i < ntiles) {
      const int nt = i % ntn, pt = i / ntn;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < lay.LRpad; k0 += M::K) {
        const typename M::frag fa = load_frag_T(sB, lay.ldN, nt * 16 + li, k0);
        const typename M::frag fb = load_frag_xw<C::R>(sXT, lay.ldK, pt * 16 + li, k0, s_w);
        acc = M::mma(fa, fb, acc);
      }
      const int kq = nt * 8 + 2 * g;
      const float2 r0 = s_crot[kq], r1 = s_crot[kq + 1];
      const float v0 = d * stt[m][0] + acc[0], v1 = d * stt[m][1] + acc[1];
      const float v2 = d * stt[m][2] + acc[2], v3 = d * stt[m][3] + acc[3];
      stt[m][0] = r0.x * v0 - r0.y * v1;
      stt[m][1] = r0.y * v0 + r0.x * v1;
      stt[m][2] = r1.x * v2 - r1.y * v3;
      stt[m][3] = r1.y * v2 + r1.x * v3;
    }
  }
}

// State tiles -> LDS copy [P][ldN] in the storage type (the B operand of the
// inter-chunk MFMA).
template <class C>
__device__ __forceinline__ void state_to_lds(const PrefillArgs& a, const ChunkLayout& lay,
                                             const f32x4 (&stt)[kMaxStTiles], unsigned char* smem) {
  using T = typename C::T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int ntn = a.N / 16, ntiles = ntn * (C::P / 16);
  T* sG = reinterpret_cast<T*>(smem + lay.off_G);
#pragma unroll
  for (int m = 0; m < kMaxStTiles; ++m) {
    const int i = wave + m * kW;
    if (i < ntiles) {
      const int nt = i % ntn, pt = i / ntn;
      T* dst = sG + (pt * 16 + li) * lay.ldN + nt * 16 + 4 * g;
      if constexpr (sizeof(T) == 2) {
        const bf16x4 v = {from_f32<bf16>(stt[m][0]), from_f32<bf16>(stt[m][1]),
                          from_f32<bf16>(stt[m][2]), from_f32<bf16>(stt[m][3])};
        *reinterpret_cast<bf16x4*>(dst) = v;
      } else {
        *reinterpret_cast<f32x4*>(dst) = stt[m];
      }
    }
  }
}

// cs, gamma, omega of the tokens of chunk rows row0 .. row0+3 (row0 a
// multiple of 4), as whole-vector LDS reads.
template <int R>
__device__ __forceinline__ void key_scalars4(const float* s_cs, const float* s_gam,
                                             const float* s_om, int row0, float (&cs)[4],
                                             float (&ga)[4], float (&om)[4]) {
  if constexpr (R == 1) {
    const float4 c = *reinterpret_cast<const float4*>(s_cs + row0);
    const float4 g = *reinterpret_cast<const float4*>(s_gam + row0);
    const float4 o = *reinterpret_cast<const float4*>(s_om + row0);
    cs[0] = c.x; cs[1] = c.y; cs[2] = c.z; cs[3] = c.w;
    ga[0] = g.x; ga[1] = g.y; ga[2] = g.z; ga[3] = g.w;
    om[0] = o.x; om[1] = o.y; om[2] = o.z; om[3] = o.w;
  } else if constexpr (R == 2) {
    const float2 c = *reinterpret_cast<const float2*>(s_cs + row0 / 2);
    const float2 g = *reinterpret_cast<const float2*>(s_gam + row0 / 2);
    const float2 o = *reinterpret_cast<const float2*>(s_om + row0 / 2);
    cs[0] = cs[1] = c.x; cs[2] = cs[3] = c.y;
    ga[0] = ga[1] = g.x; ga[2] = ga[3] = g.y;
    om[0] = om[1] = o.x; om[2] = om[3] = o.y;
  } else {
    const float c = s_cs[row0 / 4], g = s_gam[row0 / 4], o = s_om[row0 / 4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cs[j] = c;
      ga[j] = g;
      om[j] = o;
    }
  }
}

// y of one chunk: units (query block qb, p-group pg) over the waves.
template <class C>
__device__ __forceinline__ void chunk_output(const PrefillArgs& a, const ChunkLayout& lay,
                                             const Seq& s, int t0, int len,
                                             const unsigned char* smem) {
  using T = typename C::T;
  using M = Mfma<T>;
  constexpr int R = C::R, P = C::P;
  constexpr int NPT = P / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int N = a.N;
  const T* sC = reinterpret_cast<const T*>(smem + lay.off_C);
  const T* sB = reinterpret_cast<const T*>(smem + lay.off_B);
  const T* sXT = reinterpret_cast<const T*>(smem + lay.off_XT);
  const T* sG = reinterpret_cast<const T*>(smem + lay.off_G);
  const float* s_cs = reinterpret_cast<const float*>(smem + lay.off_cs);
  const float* s_gam = reinterpret_cast<const float*>(smem + lay.off_gam);
  const float* s_om = reinterpret_cast<const float*>(smem + lay.off_om);
  T* ybase = static_cast<T*>(a.y) + (((size_t)s.b * a.T + t0) * a.H + s.h) * R * P + li;
  const size_t ytok = (size_t)a.H * R * P;  // stride between tokens in y
  const int nqb = lay.LR / 16;
  int npg = 1;
  while (npg < NPT && nqb * npg * 2 <= kW) npg *= 2;
  const int ppg = NPT / npg;
  const int nunits = nqb * npg;

  for (int unit = wave; unit < nunits; unit += kW) {
    const int qb = unit / npg, pg = unit % npg;
    const int p_lo = pg * ppg, p_hi = p_lo + ppg;
    f32x4 acc[NPT];
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // inter-chunk term: C~ G_c, rows scaled by exp(cs_t)
    for (int n0 = 0; n0 < N; n0 += M::K) {
      const typename M::frag fa = M::load(sC, lay.ldN, qb * 16 + li, n0);
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt)
        if (pt >= p_lo && pt < p_hi) {
          const typename M::frag fb = M::load(sG, lay.ldN, pt * 16 + li, n0);
          acc[pt] = M::mma(fa, fb, acc[pt]);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sc = __expf(s_cs[(qb * 16 + 4 * g + j) / R]);
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) acc[pt][j] *= sc;
    }

    // intra-chunk term over key blocks up to the diagonal
    const int tq = (qb * 16 + li) / R;
    const float csq = s_cs[tq];
    constexpr int KB = (sizeof(T) == 2) ? 2 : 1;  // 16-row key blocks per step
    for (int kb = 0; kb * 16 <= qb * 16 + 15; kb += KB) {
      f32x4 sc[KB];
#pragma unroll
      for (int i = 0; i < KB; ++i) sc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int n0 = 0; n0 < N; n0 += M::K) {
        const typename M::frag fq = M::load(sC, lay.ldN, qb * 16 + li, n0);
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          const typename M::frag fk = M::load(sB, lay.ldN, (kb + i) * 16 + li, n0);
          sc[i] = M::mma(fk, fq, sc[i]);  // rows = keys, cols = queries
        }
      }
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        float kcs[4], kga[4], kom[4];
        key_scalars4<R>(s_cs, s_gam, s_om, (kb + i) * 16 + 4 * g, kcs, kga, kom);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tk = ((kb + i) * 16 + 4 * g + j) / R;
          float w = 0.f;
          if (tk < tq)
            w = __expf(csq - kcs[j]) * (kga[j] + kom[j]);
          else if (tk == tq)
            w = kga[j];
          sc[i][j] *= w;
        }
      }
      if constexpr (sizeof(T) == 2) {
        bf16x8 fa;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          fa[j] = from_f32<bf16>(sc[0][j]);
          fa[4 + j] = from_f32<bf16>(sc[1][j]);
        }
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt)
          if (pt >= p_lo && pt < p_hi) {
            const bf16* xr = reinterpret_cast<const bf16*>(sXT) + (pt * 16 + li) * lay.ldK;
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(xr + kb * 16 + 4 * g);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(xr + (kb + 1) * 16 + 4 * g);
            bf16x8 fb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              fb[j] = lo[j];
              fb[4 + j] = hi[j];
            }
            acc[pt] = Mfma<bf16>::mma(fa, fb, acc[pt]);
          }
      } else {
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt)
          if (pt >= p_lo && pt < p_hi) {
            const float* xr = reinterpret_cast<const float*>(sXT) + (pt * 16 + li) * lay.ldK;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[pt] = Mfma<float>::mma(sc[0][j], xr[kb * 16 + 4 * g + j], acc[pt]);
          }
      }
    }

#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = qb * 16 + 4 * g + j;
      const int u = row / R;
      if (u < len) {
        T* yrow = ybase + (size_t)u * ytok + (row % R) * P;
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt)
          if (pt >= p_lo && pt < p_hi) yrow[pt * 16] = from_f32<T>(acc[pt][j]);
      }
    }
  }
}

// One chunk of phase 1: commit chunk c, prefetch chunk nc (with C if kNextC),
// advance the zero-entry state of the segment.
template <class C, bool kNextC>
__device__ __forceinline__ void local_step(const PrefillArgs& a, const ChunkLayout& lay,
                                           const Seq& s, const Maps& mp, int c, int nc, float Ah,
                                           Stage<C>& stg, f32x4 (&stt)[kMaxStTiles],
                                           float& seg_logdecay, unsigned char* smem) {
  __syncthreads();  // previous chunk's LDS reads are done
  commit_stage<C, false>(a, s, mp, lay, c, stg, smem);
  __syncthreads();
  issue_loads<C, kNextC>(a, s, mp, nc, stg);
  const int t0 = c * a.L, len = min(a.L, a.T - t0);
  chunk_scalars(a, lay, len, t0, Ah, smem);
  chunk_rotate<C, false, true>(a, lay, len, smem);
  const float lc = reinterpret_cast<const float*>(smem + lay.off_cs)[a.L - 1];
  seg_logdecay += lc;
  state_update<C>(a, lay, __expf(lc), stt, smem);
}

// One chunk of phase 3: commit chunk c, prefetch chunk c + 1 (kMore), write
// its outputs, advance the state to the next chunk.
template <class C, bool kMore>
__device__ __forceinline__ void output_step(const PrefillArgs& a, const ChunkLayout& lay,
                                            const Seq& s, const Maps& mp, int c, float Ah,
                                            Stage<C>& stg, f32x4 (&stt)[kMaxStTiles],
                                            unsigned char* smem) {
  __syncthreads();
  commit_stage<C, true>(a, s, mp, lay, c, stg, smem);
  state_to_lds<C>(a, lay, stt, smem);
  __syncthreads();
  if constexpr (kMore) issue_loads<C, true>(a, s, mp, c + 1, stg);
  const int t0 = c * a.L, len = min(a.L, a.T - t0);
  chunk_scalars(a, lay, len, t0, Ah, smem);
  chunk_rotate<C, true, false>(a, lay, len, smem);
  chunk_output<C>(a, lay, s, t0, len, smem);
  if constexpr (kMore)
    state_update<C>(a, lay, __expf(reinterpret_cast<const float*>(smem + lay.off_cs)[a.L - 1]),
                    stt, smem);
}

// ---------------------------------------------------------------------------
template <class C>
__global__ void __launch_bounds__(kThreads) prefill_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int P = C::P;
  const ChunkLayout lay = chunk_layout(a.L, C::R, a.N, P, C::es);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;

  // the ticket passes through the (not yet used) angle-partial area of LDS
  int* s_ticket = reinterpret_cast<int*>(smem + lay.off_part);
  if (tid == 0) *s_ticket = atomicAdd(a.ticket, 1);
  __syncthreads();
  const int ticket = *s_ticket;
  const int BH = a.nb * a.H;
  Seq s;
  s.seg = ticket / BH;
  s.bh = ticket % BH;
  s.b = s.bh / a.H;
  s.h = s.bh % a.H;
  s.c0 = s.seg * a.K;
  s.c1 = min(a.nC, s.c0 + a.K);
  const float Ah = a.A[s.h];
  const int npair = a.N / 2;
  const int ntn = a.N / 16, ntiles = ntn * (P / 16);
  const Maps mp = {vec_map(a.N / C::vec), vec_map(P / C::vec), vec_map(a.N / 8)};
  double* s_sang = reinterpret_cast<double*>(smem + lay.off_sang);
  float2* s_srot = reinterpret_cast<float2*>(smem + lay.off_srot);

  for (int i = tid; i < npair; i += kThreads) s_sang[i] = 0.0;

  f32x4 stt[kMaxStTiles];
#pragma unroll
  for (int m = 0; m < kMaxStTiles; ++m) stt[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- phase 1: local exit state of the segment --------------------------
  // Each step prefetches the next chunk; the last one prefetches the first
  // chunk again, with C, for phase 3.
  Stage<C> stg;  // next chunk's B, (C,) x, theta, dt, lam
  issue_loads<C, false>(a, s, mp, s.c0, stg);
  float seg_logdecay = 0.f;
  for (int c = s.c0; c + 1 < s.c1; ++c)
    local_step<C, false>(a, lay, s, mp, c, c + 1, Ah, stg, stt, seg_logdecay, smem);
  local_step<C, true>(a, lay, s, mp, s.c1 - 1, s.c0, Ah, stg, stt, seg_logdecay, smem);

  // ---- phase 2: chain ------------------------------------------------------
  __syncthreads();
  for (int kp = tid; kp < npair; kp += kThreads) {
    float sn, cn;
    sincosf(static_cast<float>(s_sang[kp]), &sn, &cn);
    s_srot[kp] = make_float2(cn, sn);
  }
  const float segD = __expf(seg_logdecay);
  f32x4 ent[kMaxStTiles];
#pragma unroll
  for (int m = 0; m < kMaxStTiles; ++m) ent[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (s.seg > 0) {
    if (tid == 0) {
      int spins = 0;
      while (__hip_atomic_load(a.flags + s.bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
             s.seg) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > kSpinLimit) {
          __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    __syncthreads();
    const float* src = a.ring + ((size_t)s.bh * 2 + ((s.seg - 1) & 1)) * a.N * P;
#pragma unroll
    for (int m = 0; m < kMaxStTiles; ++m) {
      const int i = wave + m * kW;
      if (i < ntiles) {
        const int nt = i % ntn, pt = i / ntn;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          ent[m][j] = __hip_atomic_load(src + (size_t)(nt * 16 + 4 * g + j) * P + pt * 16 + li,
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  } else {
    __syncthreads();
  }
  // exit state = R(Phi_seg) (D_seg * entry) + local
  const bool last = s.seg == a.nSeg - 1;
  float* dst = a.ring + ((size_t)s.bh * 2 + (s.seg & 1)) * a.N * P;
#pragma unroll
  for (int m = 0; m < kMaxStTiles; ++m) {
    const int i = wave + m * kW;
    if (i < ntiles) {
      const int nt = i % ntn, pt = i / ntn;
      const int kq = nt * 8 + 2 * g;
      const float2 r0 = s_srot[kq], r1 = s_srot[kq + 1];
      f32x4 e;
      const float v0 = segD * ent[m][0], v1 = segD * ent[m][1];
      const float v2 = segD * ent[m][2], v3 = segD * ent[m][3];
      e[0] = r0.x * v0 - r0.y * v1 + stt[m][0];
      e[1] = r0.y * v0 + r0.x * v1 + stt[m][1];
      e[2] = r1.x * v2 - r1.y * v3 + stt[m][2];
      e[3] = r1.y * v2 + r1.x * v3 + stt[m][3];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t off = (size_t)(nt * 16 + 4 * g + j) * P + pt * 16 + li;
        if (!last)
          __hip_atomic_store(dst + off, e[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else if (a.h_final)
          a.h_final[(size_t)s.bh * a.N * P + off] = e[j];
      }
    }
  }
  if (!last) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's ring stores have completed
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(a.flags + s.bh, s.seg + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int m = 0; m < kMaxStTiles; ++m) stt[m] = ent[m];

  // ---- phase 3: outputs from the true entry state -------------------------
  for (int c = s.c0; c + 1 < s.c1; ++c) output_step<C, true>(a, lay, s, mp, c, Ah, stg, stt, smem);
  output_step<C, false>(a, lay, s, mp, s.c1 - 1, Ah, stg, stt, smem);
}

__global__ void reset_kernel(int* flags, int n) {
  for (int i = threadIdx.x; i < n + 2; i += blockDim.x) flags[i] = 0;
}

template <class C>
hipError_t launch_cfg(const PrefillArgs& a, hipStream_t stream) {
  const ChunkLayout lay = chunk_layout(a.L, C::R, a.N, C::P, C::es);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<C>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lay.total);
  if (e != hipSuccess) return e;
  const int BH = a.nb * a.H;
  // flags[BH], ticket and err are contiguous in the workspace
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(256), 0, stream, a.flags, BH);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_kernel<C>), dim3(BH * a.nSeg), dim3(kThreads), lay.total, stream,
                     a);
  return hipGetLastError();
}

template <typename T, int R, int P>
hipError_t launch_trp(const PrefillArgs& a, hipStream_t stream) {
  const int mv = chunk_stage_vectors(a.L, R, a.N, P, sizeof(T));
  return mv <= 2 ? launch_cfg<Cfg<T, R, P, 2>>(a, stream) : launch_cfg<Cfg<T, R, P, 4>>(a, stream);
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

__global__ void fill_zero_kernel(float* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace

// Chunks per segment: enough segments to give about four workgroups per CU
// across all sequences.
int prefill_segment_chunks(int nb, int H, int nC) {
  const long units = (long)nb * H;
  const long target = 1024;
  long k = (nC * units + target - 1) / target;
  if (k < 1) k = 1;
  if (k > nC) k = nC;
  return (int)k;
}

hipError_t launch_prefill(const PrefillArgs& a, m3_dtype dtype, hipStream_t stream) {
  if (a.nb == 0) return hipSuccess;
  if (a.T == 0) {
    if (!a.h_final) return hipSuccess;
    const size_t n = (size_t)a.nb * a.H * a.N * a.P;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       a.h_final, n);
    return hipGetLastError();
  }
  return dtype == M3_BF16 ? launch_t<bf16>(a, stream) : launch_t<float>(a, stream);
}

}  // namespace m3
