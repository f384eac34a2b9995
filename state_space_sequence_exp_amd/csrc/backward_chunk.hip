// backward_chunk.hip -- gradients of the recurrence by chunks, with the
// contractions on the matrix cores (state size N = 64, head dimension P = 64,
// rank R of 1, 2 or 4; other shapes take the token walks of backward.hip).
//
// The forward pass in the chunked form (Mamba-3 paper summary, Proposition 1,
// the trapezoid rule; explainer, "second improvement", the rotation folded
// into B and C; paper summary, item 3, rank R): within a chunk of L tokens
// (rows (t, r), LR = L R = 64), with angles phi_t = sum_{s<=t} dt_s theta_s
// restarting at the chunk, B~ = R(phi)^T B, C~ = R(phi)^T C,
// cs_t = sum_{s<=t} A dt_s, gamma_t = lam_t dt_t, omega_t = (1 - lam_{t+1})
// dt_{t+1} (the next token's trapezoid weight, across the chunk end too) and
// G the chunk's entry state (unrotated, its previous token's term included):
//
//   y_t     = e^{cs_t} C~_t^T G + sum_{u<=t} W[t,u] (C~_t . B~_u) x_u,
//             W[t,u] = e^{cs_t - cs_u} (gamma_u + [u<t] omega_u)
//   G_next  = R(phi_{L-1}) (e^{cs_{L-1}} G + sum_u V_u B~_u x_u^T),
//             V_u = e^{cs_{L-1} - cs_u} (gamma_u + omega_u)
//
// Reverse mode, with E the adjoint of G_next and E~ = R(phi_{L-1})^T E:
//
//   dG       = sum_t e^{cs_t} C~_t dy_t^T + e^{cs_{L-1}} E~        (the chain)
//   dx       = (W o C~B~^T)^T dY + diag(V) B~ E~
//   dB~      = (W o dY X^T)^T C~ + diag(V) X E~^T
//   dC~      = (W o dY X^T) B~ + diag(e^{cs}) dY G^T
//
// and the scalars from dW = (C~B~^T) o (dY X^T): row and column sums give
// the gradients of cs, gamma and omega; the rotations give those of phi
// (dB~_0 B~_1 - dB~_1 B~_0 per pair, likewise for C~, plus the exit
// rotation's term), whose suffix sums over the chunk are the gradients of
// dt theta.  Four launches:
//   bwc_local_kernel   per chunk: S_c = sum_u V_u B~_u x_u^T and
//                      D_c = sum_t e^{cs_t} C~_t dy_t^T (MFMA), the chunk's
//                      decay and rotation;
//   bwc_chain_kernel   per sequence, over its chunks: the entry states G_c
//                      forward and the exit adjoints dG_{c+1} backward;
//   bwc_grads_kernel   per chunk: the six products above and their
//                      epilogues (MFMA), every per-element gradient, and per
//                      token the partial scalar gradients;
//   bwc_final_kernel   per token: dt and lam from the partials (the omega
//                      term of a token comes from the chunk of the token
//                      before it); per head: dA from the chunks' partials, in
//                      a fixed order.
// Every sum runs in a fixed order, so results repeat bit for bit.
//
// Products use v_mfma_f32_16x16x4_f32 (float32 throughout, the gradients'
// parity bound being float32's).  The LDS tiles are 64 x 64 floats, row-major
// with the columns of row r XOR-swizzled by ((r & 3) << 4) | (((r >> 2) & 3)
// << 2): an MFMA operand read, 16 lanes along rows and 4 along columns or the
// other way round, then touches 64 distinct banks either way, so every product
// reads both orientations of a tile from one copy.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

constexpr int kBT = 512;  // threads of a chunk workgroup (8 waves)

// The thread index, opaque to the compiler at each use, so that the gradient
// kernel's loop over chunks does not hoist lane-dependent LDS addresses out
// of the loop and hold them in registers across it.
__device__ __forceinline__ int ltid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ int tix(int r, int c) {
  return r * 64 + (c ^ (((r & 3) << 4) | (((r >> 2) & 3) << 2)));
}
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Two products over k in [kb, ke) (multiples of 16, uniform over the wave):
// acc0 += A0 B0 and acc1 += A1 B1, where op(k, a0, b0, a1, b1) reads this
// lane's four operands of the k-step at k (rows / columns k + g).  The
// operands of the next 16 k (four steps) are requested before the current
// four steps are multiplied, so the LDS latency hides behind eight MFMAs.
template <class F>
__device__ __forceinline__ void mma_pipe2(f32x4& acc0, f32x4& acc1, int kb, int ke, F op) {
  if (kb >= ke) return;
  float a0[4], b0[4], a1[4], b1[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) op(kb + 4 * s, a0[s], b0[s], a1[s], b1[s]);
  for (int k = kb; k < ke; k += 16) {
    float na0[4], nb0[4], na1[4], nb1[4];
    const bool more = k + 16 < ke;
    if (more) {
#pragma unroll
      for (int s = 0; s < 4; ++s) op(k + 16 + 4 * s, na0[s], nb0[s], na1[s], nb1[s]);
    }
    // keep those reads ahead of the products (the scheduler would otherwise
    // sink each read next to its MFMA and wait on it there)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      acc0 = mma4(a0[s], b0[s], acc0);
      acc1 = mma4(a1[s], b1[s], acc1);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (more) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        a0[s] = na0[s];
        b0[s] = nb0[s];
        a1[s] = na1[s];
        b1[s] = nb1[s];
      }
    }
  }
}

// LDS (float offsets).  The four input tiles come first in both kernels.
constexpr int oC = 0, oB = 4096, oX = 8192, oDY = 12288;
// gradient kernel
constexpr int oM1 = 16384, oM2 = 20480, oG = 24576, oE = 28672;
constexpr int oRevG = 32768, oDphi = 34816, oScG = 36864;
// local kernel
constexpr int oRevL = 16384, oScL = 18432;
// scalar block (offsets within it)
constexpr int sDt = 0, sLam = 68, sCs = 136, sGam = 200, sOm = 264, sEcs = 328, sV = 392,
              sExitCS = 456, sExitT = 520, sMisc = 552, sDeP = 584, sDvP = 712, sRowP = 840,
              sColI = 968, sColS = 1224, sThp = 1480, sZ = 1544, sDg = 1608, sDo = 1672,
              kScGrad = 1736, kScLocal = 584;
constexpr size_t kLdsGrads = (size_t)(oScG + kScGrad) * 4;
// local: its scalars, then 16 x 32 doubles of angle partial sums
constexpr size_t kLdsLocal = (size_t)(oScL + kScLocal) * 4 + 16 * 32 * 8;

// What both chunk kernels stage: the B, C, x, dy tiles, the per-token
// scalars and the chunk's angles.  Thread (k = tid & 31, grp = tid >> 5)
// owns pair k of tokens grp * TPG .. + TPG - 1 for the angle scans and keeps
// their theta in th[].
template <int R>
struct ChunkGeo {
  static constexpr int L = 64 / R;     // tokens of a chunk
  static constexpr int TPG = L / 16;   // tokens per angle group
};

// Phase 2 (after a barrier): each thread's angle partial sum, in double.
template <int R>
__device__ __forceinline__ void stage_angle_parts(const float* sc, const float (&th)[4], double* part) {
  constexpr int TPG = ChunkGeo<R>::TPG;
  const int tid = ltid(), k = tid & 31, grp = tid >> 5;
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < TPG; ++j) s += (double)sc[sDt + grp * TPG + j] * (double)th[j];
  part[grp * 32 + k] = s;
}

// Phase 3 (after a barrier): the running angles as revolutions (the
// hardware sine / cosine input), the chunk's total rotation (accurate
// sincos of the reduced double angle, which the chain multiplies over the
// whole sequence), and (wave 0) the per-token scalars.
template <int R>
__device__ __forceinline__ void stage_angles_scalars(const BackwardArgs& a, int hh, const float (&th)[4],
                                                     const double* part, float* rev, float* sc) {
  constexpr int L = ChunkGeo<R>::L, TPG = ChunkGeo<R>::TPG;
  const int tid = ltid(), k = tid & 31, grp = tid >> 5;
  // the sums of the groups before this one, in order, requested five at a
  // time (one at a time, the later groups waited out fifteen LDS round trips)
  constexpr int NG = kBT / 32;
  double phi = 0.0;
#pragma unroll
  for (int g0 = 0; g0 < NG - 1; g0 += 5) {
    double v[5];
#pragma unroll
    for (int q = 0; q < 5; ++q) v[q] = g0 + q < NG - 1 ? part[(g0 + q) * 32 + k] : 0.0;
#pragma unroll
    for (int q = 0; q < 5; ++q)
      if (g0 + q < NG - 1 && g0 + q < grp) phi += v[q];
  }
#pragma unroll
  for (int j = 0; j < TPG; ++j) {
    const int t = grp * TPG + j;
    phi += (double)sc[sDt + t] * (double)th[j];
    const double rv = phi * 0.15915494309189535;
    rev[t * 32 + k] = (float)(rv - floor(rv));
    if (t == L - 1) {
      const double red = phi - 6.283185307179586 * rint(rv);
      float sn, cn;
      sincosf((float)red, &sn, &cn);
      sc[sExitCS + k] = cn;
      sc[sExitCS + 32 + k] = sn;
    }
  }
  if (tid < 64) {
    const int t = tid;
    const float Ah = a.A[hh];
    const float d = t < L ? sc[sDt + t] : 0.f;
    // inclusive scan over the wave (DPP; the whole of wave 0 runs this)
    const float cs = wave_incl_scan(Ah * d), csl = wave_read_lane(cs, L - 1);
    if (t < L) {
      const float gam = sc[sLam + t] * d;
      const float om = (1.f - sc[sLam + t + 1]) * sc[sDt + t + 1];
      sc[sCs + t] = cs;
      sc[sGam + t] = gam;
      sc[sOm + t] = om;
      sc[sEcs + t] = __expf(cs);
      sc[sV + t] = __expf(csl - cs) * (gam + om);
    }
  }
}

// Phase 4 (after a barrier): B and C rows rotated in place into B~, C~.
template <int R>
__device__ __forceinline__ void stage_rotate(float* sm, const float* rev) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = ltid() + kBT * q, row = idx >> 5, k = idx & 31;
    const float rv = rev[(row / R) * 32 + k];
    const float cn = __builtin_amdgcn_cosf(rv), sn = __builtin_amdgcn_sinf(rv);
    float2* pb = reinterpret_cast<float2*>(sm + oB + tix(row, 2 * k));
    float2* pc = reinterpret_cast<float2*>(sm + oC + tix(row, 2 * k));
    const float2 b = *pb, cc = *pc;
    *pb = make_float2(cn * b.x + sn * b.y, cn * b.y - sn * b.x);
    *pc = make_float2(cn * cc.x + sn * cc.y, cn * cc.y - sn * cc.x);
  }
}

// ---- a chunk's inputs as raw registers (the gradient pass fetches the next
// chunk's while it works on the current one) --------------------------------
typedef __amdgpu_buffer_rsrc_t brsrc;
__device__ __forceinline__ brsrc mkr(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// This thread's share of one chunk's inputs: 8 storage elements of each of
// the C, B, x and dy tiles (row tid / 8, columns 8 (tid % 8) ..), dt and lam
// of token tid (tid <= L), theta of pair tid % 32 for its TPG tokens.  Every
// load is a range-checked buffer load (rows past the sequence read as
// zeros), so nothing waits on a value before it is used.
template <typename T>
struct ChunkIn {
  static constexpr int kV = sizeof(T) / 2;  // 16-byte vectors per 8 elements
  u32x4 t[4][kV];
  uint32_t dt, lam, th[4];
};

template <typename T, int R>
__device__ __forceinline__ void chunk_fetch(const BackwardArgs& a, int ci, int nC, ChunkIn<T>& in) {
  constexpr int L = ChunkGeo<R>::L, TPG = ChunkGeo<R>::TPG;
  constexpr uint32_t es = sizeof(T);
  const int tid = ltid(), row = tid >> 3, c0 = (tid & 7) * 8;
  const int unit = ci / nC, c = ci - unit * nC, b = unit / a.H, hh = unit - b * a.H;
  const int t0 = c * L, len = min(L, a.T - t0);
  const size_t tok0 = ((size_t)b * a.T + t0) * a.H + hh;
  const uint32_t stride = (uint32_t)a.H * R * 64 * es;  // bytes from one token's rows to the next
  const uint32_t range = (uint32_t)(len - 1) * stride + R * 64 * es;
  const uint32_t off = (uint32_t)(row / R) * stride + (uint32_t)((row % R) * 64 + c0) * es;
  const void* src[4] = {a.C, a.B, a.x, a.dy};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const brsrc r = mkr(static_cast<const unsigned char*>(src[q]) + tok0 * R * 64 * es, range);
#pragma unroll
    for (int v = 0; v < ChunkIn<T>::kV; ++v)
      in.t[q][v] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 16 * v), 0, 0);
  }
  const int nsc = min(L + 1, a.T - t0);  // dt, lam of tokens t0 .. t0 + L
  const brsrc rd = mkr(a.dt + tok0, (uint32_t)(nsc - 1) * a.H * 4 + 4);
  const brsrc rl = mkr(a.lam + tok0, (uint32_t)(nsc - 1) * a.H * 4 + 4);
  const uint32_t so = (uint32_t)min(tid, L + 1) * a.H * 4;
  in.dt = __builtin_amdgcn_raw_buffer_load_b32(rd, (int)so, 0, 0);
  in.lam = __builtin_amdgcn_raw_buffer_load_b32(rl, (int)so, 0, 0);
  const uint32_t tstride = (uint32_t)a.H * 32 * 4;
  const brsrc rt = mkr(a.theta + tok0 * 32, (uint32_t)(len - 1) * tstride + 128);
  const int k = tid & 31, grp = tid >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    in.th[j] = j < TPG ? __builtin_amdgcn_raw_buffer_load_b32(
                             rt, (int)((uint32_t)(grp * TPG + j) * tstride + k * 4), 0, 0)
                       : 0u;
}

// The fetched tiles into LDS as float, dt and lam into the scalar block,
// theta into th[].
template <typename T, int R>
__device__ __forceinline__ void chunk_commit(const ChunkIn<T>& in, float* sm, float* sc,
                                             float (&th)[4]) {
  constexpr int L = ChunkGeo<R>::L;
  const int tid = ltid(), row = tid >> 3, c0 = (tid & 7) * 8;
  const int toff[4] = {oC, oB, oX, oDY};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v[8];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(in.t[q][0][e] << 16);
        v[2 * e + 1] = __uint_as_float(in.t[q][0][e] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = __uint_as_float(in.t[q][0][e]);
        v[4 + e] = __uint_as_float(in.t[q][1][e]);
      }
    }
    *reinterpret_cast<float4*>(sm + toff[q] + tix(row, c0)) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(sm + toff[q] + tix(row, c0 + 4)) = make_float4(v[4], v[5], v[6], v[7]);
  }
  if (tid <= L) {
    sc[sDt + tid] = __uint_as_float(in.dt);
    sc[sLam + tid] = __uint_as_float(in.lam);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) th[j] = __uint_as_float(in.th[j]);
}

// ---- local pass ---------------------------------------------------------------
// Per (sequence, head, chunk): S_c into slot c + 1 of the entry states, D_c
// into slot c of the adjoints, and the chunk's decay and rotation.  The
// workgroups are persistent over the chunks (chunk ci, ci + gridDim.x, ...),
// with the next chunk's inputs requested into registers as soon as the
// current chunk's are in the LDS, so their latency hides behind this
// chunk's work.  Registers are held to 128 a lane so that two workgroups
// share a CU (the LDS holds two): 266.5 against 275.7 us for the whole
// backward at the SISO bench shape with one workgroup per CU, and 277.4 us
// before, with one workgroup per chunk.
template <typename T, int R>
__global__ void __launch_bounds__(kBT) __attribute__((amdgpu_waves_per_eu(4)))
bwc_local_kernel(BackwardArgs a, int nC) {
  extern __shared__ __align__(16) float sm[];
  float* sc = sm + oScL;
  float* rev = sm + oRevL;
  double* part = reinterpret_cast<double*>(sm + oScL + kScLocal);
  const int nchunk = a.nb * a.H * nC;
  ChunkIn<T> in;
  chunk_fetch<T, R>(a, blockIdx.x, nC, in);
  for (int ci = blockIdx.x; ci < nchunk; ci += gridDim.x) {
    const int unit = ci / nC, c = ci - unit * nC;
    float th[4];
    __syncthreads();  // every read of the previous chunk's LDS is done
    chunk_commit<T, R>(in, sm, sc, th);
    if (ci + (int)gridDim.x < nchunk) chunk_fetch<T, R>(a, ci + gridDim.x, nC, in);
    __syncthreads();
    stage_angle_parts<R>(sc, th, part);
    __syncthreads();
    stage_angles_scalars<R>(a, unit % a.H, th, part, rev, sc);
    __syncthreads();
    stage_rotate<R>(sm, rev);
    __syncthreads();

    const int tl = ltid(), lane = tl & 63, w = tl >> 6, i = lane & 15, g = lane >> 4;
    const int m0 = (w >> 1) * 16;
    constexpr int NP = 64 * 64;
    float* Sout = a.hs + ((size_t)unit * (nC + 1) + c + 1) * NP;
    float* Dout = a.gs + ((size_t)unit * nC + c) * NP;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int n0 = (2 * (w & 1) + q) * 16;
      f32x4 s = {0.f, 0.f, 0.f, 0.f}, d = {0.f, 0.f, 0.f, 0.f};
      mma_pipe2(s, d, 0, 64, [&](int k, float& a0, float& b0, float& a1, float& b1) {
        const int kr = k + g, tk = kr / R;
        a0 = sm[oB + tix(kr, m0 + i)];
        b0 = sc[sV + tk] * sm[oX + tix(kr, n0 + i)];
        a1 = sm[oC + tix(kr, m0 + i)];
        b1 = sc[sEcs + tk] * sm[oDY + tix(kr, n0 + i)];
      });
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = m0 + 4 * g + j;
        Sout[n * 64 + n0 + i] = s[j];
        Dout[n * 64 + n0 + i] = d[j];
      }
    }
    constexpr int L = ChunkGeo<R>::L;
    float* cs_out = a.dseg + ((size_t)unit * nC + c) * 65;
    if (threadIdx.x < 64) cs_out[threadIdx.x] = sc[sExitCS + threadIdx.x];
    if (threadIdx.x == 64) cs_out[64] = sc[sEcs + L - 1];
  }
}

// ---- chain ----------------------------------------------------------------------
// blockIdx.y 0: entry states forward, G_{c+1} = R(Phi_c)(e_c G_c + S_c) in
// place of S_c (slot c + 1), slot 0 zero; 1: adjoints backward, slot c of
// the adjoints becomes dG_{c+1} and dG_c = D_c + e_c R(Phi_c)^T dG_{c+1}.
// Thread (k, p) of a sequence holds rows 2k, 2k + 1 of column p; chunks in
// blocks of 8 with all of a block's loads issued first.
__global__ void __launch_bounds__(256) bwc_chain_kernel(BackwardArgs a, int nC) {
  constexpr int NP = 64 * 64, kBlk = 8;
  const int unit = blockIdx.x, pidx = blockIdx.z * 256 + threadIdx.x;
  const int k = pidx >> 6, p = pidx & 63;
  const int e0i = (2 * k) * 64 + p, e1i = e0i + 64;
  const float* cs_in = a.dseg + (size_t)unit * nC * 65;
  if (blockIdx.y == 0) {
    float* Gs = a.hs + (size_t)unit * (nC + 1) * NP;
    float g0 = 0.f, g1 = 0.f;
    Gs[e0i] = 0.f;
    Gs[e1i] = 0.f;
    for (int cb = 0; cb < nC; cb += kBlk) {
      float s0[kBlk], s1[kBlk], cn[kBlk], sn[kBlk], ee[kBlk];
#pragma unroll
      for (int j = 0; j < kBlk; ++j) {
        const int c = cb + j;
        if (c < nC) {
          const float* S = Gs + (size_t)(c + 1) * NP;
          s0[j] = S[e0i];
          s1[j] = S[e1i];
          cn[j] = cs_in[(size_t)c * 65 + k];
          sn[j] = cs_in[(size_t)c * 65 + 32 + k];
          ee[j] = cs_in[(size_t)c * 65 + 64];
        }
      }
#pragma unroll
      for (int j = 0; j < kBlk; ++j) {
        const int c = cb + j;
        if (c < nC) {
          const float y0 = __builtin_fmaf(ee[j], g0, s0[j]), y1 = __builtin_fmaf(ee[j], g1, s1[j]);
          g0 = cn[j] * y0 - sn[j] * y1;
          g1 = sn[j] * y0 + cn[j] * y1;
          float* G = Gs + (size_t)(c + 1) * NP;
          G[e0i] = g0;
          G[e1i] = g1;
        }
      }
    }
  } else {
    float* Ds = a.gs + (size_t)unit * nC * NP;
    float e0 = 0.f, e1 = 0.f;
    if (a.dh_final) {
      e0 = a.dh_final[(size_t)unit * NP + e0i];
      e1 = a.dh_final[(size_t)unit * NP + e1i];
    }
    for (int cb = nC - 1; cb >= 0; cb -= kBlk) {
      float d0[kBlk], d1[kBlk], cn[kBlk], sn[kBlk], ee[kBlk];
#pragma unroll
      for (int j = 0; j < kBlk; ++j) {
        const int c = cb - j;
        if (c >= 0) {
          const float* D = Ds + (size_t)c * NP;
          d0[j] = D[e0i];
          d1[j] = D[e1i];
          cn[j] = cs_in[(size_t)c * 65 + k];
          sn[j] = cs_in[(size_t)c * 65 + 32 + k];
          ee[j] = cs_in[(size_t)c * 65 + 64];
        }
      }
#pragma unroll
      for (int j = 0; j < kBlk; ++j) {
        const int c = cb - j;
        if (c >= 0) {
          float* D = Ds + (size_t)c * NP;
          D[e0i] = e0;
          D[e1i] = e1;
          const float r0 = cn[j] * e0 + sn[j] * e1, r1 = cn[j] * e1 - sn[j] * e0;
          e0 = __builtin_fmaf(ee[j], r0, d0[j]);
          e1 = __builtin_fmaf(ee[j], r1, d1[j]);
        }
      }
    }
  }
}

// ---- gradients --------------------------------------------------------------------

// Sum over the 16 lanes of a DPP row (lanes sharing l >> 4), in every lane.
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  return v;
}
// Sum over the 4 lanes l % 16 + 16 g (g = 0 .. 3), in every lane.
__device__ __forceinline__ float sum_groups(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// The epilogue of dB~ or dC~ (one 16 x 16 tile, lane (i, g), rows m0 + 4g + j,
// column n = n0 + i): the rotation gradient of pair n / 2 (summed into the
// row's dphi entry, written when `first`), and the rotated-back gradient
// R(phi) dV~ stored to `out` (rows (token, rank) of a [B, T, H, R, 64] float
// tensor).
template <int R>
__device__ __forceinline__ void rot_epilogue(const f32x4& acc, const float* vt, const float* rev,
                                             float* dphi, bool first, float* out,
                                             const BackwardArgs& a, int b, int hh, int t0, int m0,
                                             int n0) {
  const int lane = ltid() & 63, i = lane & 15, g = lane >> 4;
  const int n = n0 + i, k = n >> 1;
  const bool even = (n & 1) == 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = m0 + 4 * g + j, t = row / R;
    const float v = acc[j];
    const float pv = __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, true));
    const float own = vt[tix(row, n)], par = vt[tix(row, n ^ 1)];
    if (even) {
      const float dp = v * par - pv * own;
      float* slot = dphi + row * 32 + k;
      *slot = first ? dp : *slot + dp;
    }
    const float rv = rev[t * 32 + k];
    const float cn = __builtin_amdgcn_cosf(rv), sn = __builtin_amdgcn_sinf(rv);
    const float o = even ? cn * v - sn * pv : sn * pv + cn * v;
    if (t0 + t < a.T)
      out[((((size_t)b * a.T + t0 + t) * a.H + hh) * R + row % R) * 64 + n] = o;
  }
}

// Persistent: workgroup j takes chunks j, j + grid, ...  With bfloat16 inputs
// the next chunk's inputs are fetched into registers once the current
// chunk's states are consumed, so they arrive during its products; float
// inputs (twice the registers) are fetched at the top of each chunk.
template <typename T, int R>
__global__ void __launch_bounds__(kBT) bwc_grads_kernel(BackwardArgs a, int nC) {
  extern __shared__ __align__(16) float sm[];
  constexpr int L = ChunkGeo<R>::L, TPG = ChunkGeo<R>::TPG;
  constexpr bool kAhead = sizeof(T) == 2;
  float* sc = sm + oScG;
  float* rev = sm + oRevG;
  float* dphi = sm + oDphi;
  const int nchunk = a.nb * a.H * nC;
  ChunkIn<T> in;
  if (kAhead) chunk_fetch<T, R>(a, blockIdx.x, nC, in);
  for (int ci = blockIdx.x; ci < nchunk; ci += gridDim.x) {
  // the thread index, opaque to the compiler in each chunk: otherwise every
  // lane-dependent LDS address of the body is hoisted out of the loop and
  // held in registers across it
  const int tid = ltid();
  const int lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;
  const int unit = ci / nC, c = ci - unit * nC;
  const int b = unit / a.H, hh = unit - b * a.H, t0 = c * L;

  // ---- staging: inputs, and the states: entry G, exit G_next, its adjoint E
  if (!kAhead) chunk_fetch<T, R>(a, ci, nC, in);
  float th[4];
  chunk_commit<T, R>(in, sm, sc, th);
  // the states (written by the chain pass just before; mostly last-level
  // cache hits): rows 2 sk, 2 sk + 1, columns sp .. sp + 3
  const int sk = tid >> 4, sp = (tid & 15) * 4;
  constexpr int NP = 64 * 64;
  const float* Gp = a.hs + ((size_t)unit * (nC + 1) + c) * NP;
  const float* Ep = a.gs + ((size_t)unit * nC + c) * NP;
  const float4 G0 = *reinterpret_cast<const float4*>(Gp + (2 * sk) * 64 + sp);
  const float4 G1 = *reinterpret_cast<const float4*>(Gp + (2 * sk + 1) * 64 + sp);
  const float4 N0 = *reinterpret_cast<const float4*>(Gp + NP + (2 * sk) * 64 + sp);
  const float4 N1 = *reinterpret_cast<const float4*>(Gp + NP + (2 * sk + 1) * 64 + sp);
  const float4 E0 = *reinterpret_cast<const float4*>(Ep + (2 * sk) * 64 + sp);
  const float4 E1 = *reinterpret_cast<const float4*>(Ep + (2 * sk + 1) * 64 + sp);
  __syncthreads();
  double* part = reinterpret_cast<double*>(sm + oM1);  // free until the products
  stage_angle_parts<R>(sc, th, part);
  __syncthreads();
  stage_angles_scalars<R>(a, hh, th, part, rev, sc);
  __syncthreads();
  stage_rotate<R>(sm, rev);
  {
    // the exit rotation's angle gradient, sum_p E[2k+1] G_next[2k] - E[2k] G_next[2k+1]
    float ex = E1.x * N0.x - E0.x * N1.x + E1.y * N0.y - E0.y * N1.y + E1.z * N0.z - E0.z * N1.z +
               E1.w * N0.w - E0.w * N1.w;
    ex = sum16(ex);
    if ((tid & 15) == 0) sc[sExitT + sk] = ex;
    // E~ = R(phi_{L-1})^T E, and <E~, G>
    const float cn = sc[sExitCS + sk], sn = sc[sExitCS + 32 + sk];
    const float4 r0 = make_float4(cn * E0.x + sn * E1.x, cn * E0.y + sn * E1.y,
                                  cn * E0.z + sn * E1.z, cn * E0.w + sn * E1.w);
    const float4 r1 = make_float4(cn * E1.x - sn * E0.x, cn * E1.y - sn * E0.y,
                                  cn * E1.z - sn * E0.z, cn * E1.w - sn * E0.w);
    *reinterpret_cast<float4*>(sm + oE + tix(2 * sk, sp)) = r0;
    *reinterpret_cast<float4*>(sm + oE + tix(2 * sk + 1, sp)) = r1;
    *reinterpret_cast<float4*>(sm + oG + tix(2 * sk, sp)) = G0;
    *reinterpret_cast<float4*>(sm + oG + tix(2 * sk + 1, sp)) = G1;
    float eg = r0.x * G0.x + r0.y * G0.y + r0.z * G0.z + r0.w * G0.w + r1.x * G1.x +
               r1.y * G1.y + r1.z * G1.z + r1.w * G1.w;
    eg = sum_groups(sum16(eg));
    if (lane == 0) sc[sMisc + w] = eg;
  }
  __syncthreads();
  // the next chunk's inputs, in flight through this chunk's products
  if (kAhead && ci + (int)gridDim.x < nchunk) chunk_fetch<T, R>(a, ci + gridDim.x, nC, in);

  const int m0 = (w >> 1) * 16;          // this wave's row tile
  const int tmax = (m0 + 15) / R;        // last token of its rows
  const int tmin = m0 / R;               // first token of its rows

  // ---- scores: S1 = C~ B~^T, S2 = dY X^T; M1 = W o S1, M2 = W o S2 and the
  // sums of dW = S1 o S2 that the scalar gradients need
  {
    float rowv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int n0 = (2 * (w & 1) + q) * 16;
      const int umin = n0 / R;
      float cI = 0.f, cS = 0.f;
      if (umin > tmax) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sm[oM1 + tix(m0 + 4 * g + j, n0 + i)] = 0.f;
          sm[oM2 + tix(m0 + 4 * g + j, n0 + i)] = 0.f;
        }
      } else {
        f32x4 s1 = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
        mma_pipe2(s1, s2, 0, 64, [&](int k, float& a0, float& b0, float& a1, float& b1) {
          a0 = sm[oC + tix(m0 + i, k + g)];
          b0 = sm[oB + tix(n0 + i, k + g)];
          a1 = sm[oDY + tix(m0 + i, k + g)];
          b1 = sm[oX + tix(n0 + i, k + g)];
        });
        const int uu = n0 + i, u = uu / R;
        const float csu = sc[sCs + u], gu = sc[sGam + u], ou = sc[sOm + u];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = m0 + 4 * g + j, t = rr / R;
          float m1 = 0.f, m2 = 0.f;
          if (u <= t) {
            const float ex = __expf(sc[sCs + t] - csu);
            const float wv = ex * (gu + (u < t ? ou : 0.f));
            const float dw = s1[j] * s2[j];
            m1 = wv * s1[j];
            m2 = wv * s2[j];
            rowv[j] += dw * wv;
            cI += dw * ex;
            if (u < t) cS += dw * ex;
          }
          sm[oM1 + tix(rr, uu)] = m1;
          sm[oM2 + tix(rr, uu)] = m2;
        }
      }
      cI = sum_groups(cI);
      cS = sum_groups(cS);
      if (g == 0) {
        sc[sColI + (w >> 1) * 64 + n0 + i] = cI;
        sc[sColS + (w >> 1) * 64 + n0 + i] = cS;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float r = sum16(rowv[j]);
      if (i == 0) sc[sRowP + (w & 1) * 64 + m0 + 4 * g + j] = r;
    }
  }
  __syncthreads();

  // ---- dC~ = diag(e^cs) dY G^T + M2 B~ ---------------------------------------------
  // The wave's two column tiles n0[0], n0[1] share the A operand.  The row
  // sums de_t = C~_t . (G dy_t) and dV_u = B~_u . (E~ x_u) come from the first
  // products of dC~ and of dB~: per row, one partial per wave of the row tile.
  const int nA = (2 * (w & 1)) * 16, nB = nA + 16;
  {
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    mma_pipe2(acc0, acc1, 0, 64, [&](int k, float& a0, float& b0, float& a1, float& b1) {
      a0 = sm[oDY + tix(m0 + i, k + g)];
      a1 = a0;
      b0 = sm[oG + tix(nA + i, k + g)];
      b1 = sm[oG + tix(nB + i, k + g)];
    });
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = m0 + 4 * g + j;
      const float de = sum16(sm[oC + tix(rr, nA + i)] * acc0[j] + sm[oC + tix(rr, nB + i)] * acc1[j]);
      if (i == 0) sc[sDeP + (w & 1) * 64 + rr] = de;
      const float e = sc[sEcs + rr / R];
      acc0[j] *= e;
      acc1[j] *= e;
    }
    mma_pipe2(acc0, acc1, 0, m0 + 16, [&](int k, float& a0, float& b0, float& a1, float& b1) {
      a0 = sm[oM2 + tix(m0 + i, k + g)];
      a1 = a0;
      b0 = sm[oB + tix(k + g, nA + i)];
      b1 = sm[oB + tix(k + g, nB + i)];
    });
    // every (row, pair) entry of dphi belongs to one lane of one wave, the
    // same in the dB~ epilogue below: written here, added to there
    rot_epilogue<R>(acc0, sm + oC, rev, dphi, true, a.dC, a, b, hh, t0, m0, nA);
    rot_epilogue<R>(acc1, sm + oC, rev, dphi, true, a.dC, a, b, hh, t0, m0, nB);
  }
  // ---- dB~ = diag(V) X E~^T + M2^T C~ -------------------------------------------------
  {
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    mma_pipe2(acc0, acc1, 0, 64, [&](int k, float& a0, float& b0, float& a1, float& b1) {
      a0 = sm[oX + tix(m0 + i, k + g)];
      a1 = a0;
      b0 = sm[oE + tix(nA + i, k + g)];
      b1 = sm[oE + tix(nB + i, k + g)];
    });
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = m0 + 4 * g + j;
      const float dv = sum16(sm[oB + tix(rr, nA + i)] * acc0[j] + sm[oB + tix(rr, nB + i)] * acc1[j]);
      if (i == 0) sc[sDvP + (w & 1) * 64 + rr] = dv;
      const float v = sc[sV + rr / R];
      acc0[j] *= v;
      acc1[j] *= v;
    }
    mma_pipe2(acc0, acc1, m0, 64, [&](int k, float& a0, float& b0, float& a1, float& b1) {
      a0 = sm[oM2 + tix(k + g, m0 + i)];
      a1 = a0;
      b0 = sm[oC + tix(k + g, nA + i)];
      b1 = sm[oC + tix(k + g, nB + i)];
    });
    rot_epilogue<R>(acc0, sm + oB, rev, dphi, false, a.dB, a, b, hh, t0, m0, nA);
    rot_epilogue<R>(acc1, sm + oB, rev, dphi, false, a.dB, a, b, hh, t0, m0, nB);
  }
  // ---- dx = diag(V) B~ E~ + M1^T dY ------------------------------------------------------
  {
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    mma_pipe2(acc0, acc1, 0, 64, [&](int k, float& a0, float& b0, float& a1, float& b1) {
      a0 = sm[oB + tix(m0 + i, k + g)];
      a1 = a0;
      b0 = sm[oE + tix(k + g, nA + i)];
      b1 = sm[oE + tix(k + g, nB + i)];
    });
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v = sc[sV + (m0 + 4 * g + j) / R];
      acc0[j] *= v;
      acc1[j] *= v;
    }
    mma_pipe2(acc0, acc1, m0, 64, [&](int k, float& a0, float& b0, float& a1, float& b1) {
      a0 = sm[oM1 + tix(k + g, m0 + i)];
      a1 = a0;
      b0 = sm[oDY + tix(k + g, nA + i)];
      b1 = sm[oDY + tix(k + g, nB + i)];
    });
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = m0 + 4 * g + j, t = rr / R;
      if (t0 + t < a.T) {
        float* o = a.dx + ((((size_t)b * a.T + t0 + t) * a.H + hh) * R + rr % R) * 64;
        o[nA + i] = acc0[j];
        o[nB + i] = acc1[j];
      }
    }
  }
  __syncthreads();

  // ---- per-token scalars --------------------------------------------------------------
  if (tid < 64) {
    const int t = tid;
    float de = 0.f, dv = 0.f, rr_ = 0.f, cI = 0.f, cS = 0.f;
    if (t < L) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = t * R + r;
        de += sc[sDeP + row] + sc[sDeP + 64 + row];
        dv += sc[sDvP + row] + sc[sDvP + 64 + row];
        rr_ += sc[sRowP + row] + sc[sRowP + 64 + row];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          cI += sc[sColI + mt * 64 + row];
          cS += sc[sColS + mt * 64 + row];
        }
      }
    }
    const float e = t < L ? sc[sEcs + t] : 0.f, V = t < L ? sc[sV + t] : 0.f;
    const float gam = t < L ? sc[sGam + t] : 0.f, om = t < L ? sc[sOm + t] : 0.f;
    float dvv = dv * V;
    for (int o = 1; o < 64; o <<= 1) dvv += __shfl_xor(dvv, o);
    float eg = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) eg += sc[sMisc + q];
    float dcs = rr_ - (gam * cI + om * cS) + de * e - dv * V;
    if (t == L - 1) dcs += dvv + eg * e;
    if (t >= L) dcs = 0.f;
    // Z_t = sum_{s >= t} dcs_s
    float z = dcs;
    for (int o = 1; o < 64; o <<= 1) {
      const float n = __shfl_down(z, o);
      if (t + o < 64) z += n;
    }
    if (t < L) {
      const float eL = __expf(sc[sCs + L - 1] - sc[sCs + t]);
      sc[sZ + t] = z;
      sc[sDg + t] = cI + dv * eL;
      sc[sDo + t] = cS + dv * eL;
    }
  }
  // the angle gradients' suffix sums over the chunk: dtheta, and each token's
  // theta term of ddt
  float* gpart = sm + oM1;  // 16 x 32 group sums (the products are done)
  {
    const int k = tid & 31, grp = tid >> 5;
    float dp[4];
    float tot = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dp[j] = 0.f;
      if (j < TPG) {
        const int t = grp * TPG + j;
#pragma unroll
        for (int r = 0; r < R; ++r) dp[j] += dphi[(t * R + r) * 32 + k];
        if (t == L - 1) dp[j] += sc[sExitT + k];
        tot += dp[j];
      }
    }
    gpart[grp * 32 + k] = tot;
    __syncthreads();
    float suf = 0.f;
    for (int g2 = 15; g2 > grp; --g2) suf += gpart[g2 * 32 + k];
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (j < TPG) {
        const int t = grp * TPG + j;
        suf += dp[j];
        const float d = sc[sDt + t];
        if (t0 + t < a.T)
          a.dtheta[(((size_t)b * a.T + t0 + t) * a.H + hh) * 32 + k] = d * suf;
        float tp = th[j] * suf;
        tp += __shfl_xor(tp, 1);
        tp += __shfl_xor(tp, 2);
        tp += __shfl_xor(tp, 4);
        tp += __shfl_xor(tp, 8);
        tp += __shfl_xor(tp, 16);
        if (k == 0) sc[sThp + t] = tp;
      }
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int t = tid, gt = t0 + t;
    const size_t ntok = (size_t)a.nb * a.T * a.H;
    float* F0 = a.dAc;
    float* F1 = F0 + ntok;
    float* F2 = F1 + ntok;
    float* dAp = F2 + ntok;  // per chunk: its tokens' share of dA
    float da = 0.f;
    if (t < L && gt < a.T) {
      const size_t tok = ((size_t)b * a.T + gt) * a.H + hh;
      const float d = sc[sDt + t], lm = sc[sLam + t], z = sc[sZ + t], dg = sc[sDg + t];
      F0[tok] = a.A[hh] * z + dg * lm + sc[sThp + t];
      F1[tok] = dg * d;
      da = d * z;
      if (gt + 1 < a.T) F2[tok + a.H] = sc[sDo + t];
    }
    for (int o = 32; o > 0; o >>= 1) da += __shfl_xor(da, o);
    if (t == 0) dAp[(size_t)unit * nC + c] = da;
  }
  __syncthreads();  // the LDS is rewritten by the next chunk
  }
}

// dt and lam of every token from the chunks' partials (one thread per
// token), and (the last H workgroups) dA[h], the head's chunk partials
// summed in a fixed order.
constexpr int kFinThreads = 256;
__global__ void __launch_bounds__(kFinThreads) bwc_final_kernel(BackwardArgs a, int nC) {
  const size_t ntok = (size_t)a.nb * a.T * a.H;
  const float* F0 = a.dAc;
  const float* F1 = F0 + ntok;
  const float* F2 = F1 + ntok;
  const float* dAp = F2 + ntok;
  const size_t ntb = (ntok + kFinThreads - 1) / kFinThreads;
  if (blockIdx.x < ntb) {
    const size_t tok = (size_t)blockIdx.x * kFinThreads + threadIdx.x;
    if (tok < ntok) {
      const bool first = ((tok / a.H) % a.T) == 0;  // no token before it: no omega term
      const float f2 = first ? 0.f : F2[tok];
      a.ddt[tok] = F0[tok] + f2 * (1.f - a.lam[tok]);
      a.dlam[tok] = F1[tok] - f2 * a.dt[tok];
    }
    return;
  }
  __shared__ float s[kFinThreads];
  const int hh = (int)(blockIdx.x - ntb);
  const int n = a.nb * nC;  // (batch, chunk) partials of head hh
  float v = 0.f;
  for (int q = threadIdx.x; q < n; q += kFinThreads) {
    const int bb = q / nC, cc = q - bb * nC;
    v += dAp[((size_t)bb * a.H + hh) * nC + cc];
  }
  s[threadIdx.x] = v;
  __syncthreads();
  for (int w = kFinThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) s[threadIdx.x] += s[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.dA[hh] = s[0];
}

template <typename T, int R>
hipError_t launch_r(const BackwardArgs& a, hipStream_t stream) {
  const int L = 64 / R, nC = (a.T + L - 1) / L;
  const unsigned units = (unsigned)a.nb * a.H;
  hipError_t e = lds_limit(reinterpret_cast<const void*>(&bwc_local_kernel<T, R>), kLdsLocal);
  if (e != hipSuccess) return e;
  e = lds_limit(reinterpret_cast<const void*>(&bwc_grads_kernel<T, R>), kLdsGrads);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 0, per_cu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  const unsigned nchunk = units * nC;
  // the local pass: as many persistent workgroups as are resident at once
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
           &per_cu, reinterpret_cast<const void*>(&bwc_local_kernel<T, R>), kBT, kLdsLocal)) !=
      hipSuccess)
    return e;
  const unsigned nlocal = (unsigned)cus * (unsigned)(per_cu > 0 ? per_cu : 1);
  hipLaunchKernelGGL((bwc_local_kernel<T, R>), dim3(nchunk < nlocal ? nchunk : nlocal), dim3(kBT),
                     kLdsLocal, stream, a, nC);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwc_chain_kernel, dim3(units, 2, 8), dim3(256), 0, stream, a, nC);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // one workgroup per CU (the LDS holds one), each over several chunks
  const unsigned ngrid = nchunk < (unsigned)cus ? nchunk : (unsigned)cus;
  hipLaunchKernelGGL((bwc_grads_kernel<T, R>), dim3(ngrid), dim3(kBT), kLdsGrads, stream, a, nC);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t ntb = ((size_t)a.nb * a.T * a.H + kFinThreads - 1) / kFinThreads;
  hipLaunchKernelGGL(bwc_final_kernel, dim3((unsigned)(ntb + a.H)), dim3(kFinThreads), 0, stream, a,
                     nC);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const BackwardArgs& a, hipStream_t stream) {
  switch (a.R) {
    case 1: return launch_r<T, 1>(a, stream);
    case 2: return launch_r<T, 2>(a, stream);
    case 4: return launch_r<T, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_backward_chunked(const BackwardArgs& a, m3_dtype dtype, hipStream_t stream) {
  if (!bw_chunked_shape(a.R, a.N, a.P) || a.nb == 0 || a.T == 0) return hipErrorInvalidValue;
  return dtype == M3_BF16 ? launch_t<bf16>(a, stream) : launch_t<float>(a, stream);
}

}  // namespace m3
