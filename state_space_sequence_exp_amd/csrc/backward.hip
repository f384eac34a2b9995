// backward.hip -- gradients of the SSM layer recurrence (reverse mode).
//
// Forward, per (batch, head), in the unrotated frame:
//   P_t = sum_r B_{t,r} x_{t,r}^T                     (N x P)
//   U_t = h_{t-1} + beta_t P_{t-1},   beta_t = (1 - lam_t) dt_t,   h_{-1} = P_{-1} = 0
//   h_t = alpha_t R(psi_t) U_t + gamma_t P_t,   alpha_t = e^{dt_t A},  gamma_t = lam_t dt_t,
//         psi_t[k] = dt_t theta_t[k]
//   y_t = C_t^T h_t
// (Mamba-3 paper summary, Proposition 1, with the complex transition as 2x2
// rotations on row pairs -- explainer, "second improvement" -- and rank-R
// products, paper summary, item 3.)
//
// Reverse mode with L = sum y.dy + sum h_{T-1}.dh_final:
//   G_t  = dL/dh_t = sum_r C_{t,r} dy_{t,r}^T + dU_{t+1}   (+ dh_final at T-1)
//   dU_t = alpha_t R_t^T G_t
//   dP_t = gamma_t G_t + beta_{t+1} dU_{t+1}
//   dB_{t,r} = dP_t x_{t,r},  dx_{t,r} = dP_t^T B_{t,r},  dC_{t,r} = h_t dy_{t,r}
//   d alpha_t = <G_t, R_t U_t>,  d psi_t[k] = alpha_t <G_t, R'(psi) U_t>_pair k
//   d gamma_t = <G_t, P_t>,  d beta_t = <dU_t, P_{t-1}>
// and the chain rule through alpha, beta, gamma, psi to dt, lam, theta, A.
//
// The kernels materialise the states: fwd_states_kernel stores every h_t
// and adj_states_kernel every G_t (one lane per (row pair, column), a time
// loop each way, inputs staged kAhead tokens ahead); token_grads_kernel
// then forms every token's gradients in parallel from h_t, h_{t-1} and G_t,
// a few consecutive tokens per workgroup
// (dU_{t+1} = G_t - sum_r C dy^T, so G_{t+1} is not read); dA_kernel sums
// dA over (batch, time) per head.  Every reduction has a fixed order, so the
// results are bitwise repeatable.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

constexpr int kScanThreads = 256;

template <typename T>
__device__ __forceinline__ float ldf(const T* p) {
  return to_f32(*p);
}

// Tokens of input staged ahead in each time loop (a register ring; the loop
// is unrolled by this much so the ring indices are static).  The ring holds
// the raw bits of raw buffer loads, converted only when the step uses them,
// so a token's loads stay in flight for kAhead steps (a conversion at load
// time, or a scalar load copied into the ring, would wait at once).
constexpr int kAhead = 8;
constexpr int kRsrcW3 = 0x00020000;  // raw buffer descriptor, gfx9 family

typedef __amdgpu_buffer_rsrc_t brsrc;
__device__ __forceinline__ brsrc mk_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcW3);
}
__device__ __forceinline__ uint32_t bld32(brsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t bld16(brsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ void bst32(float v, brsrc r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)off, 0, 0);
}

// sin and cos of one token's angle dt * theta (small): reduced to revolutions
// and taken by the hardware sine / cosine, which read no table (a library
// sincos would load one and make the loop wait for every load in flight).
__device__ __forceinline__ void sincos_step(float ang, float& sn, float& cn) {
  const float r = __builtin_amdgcn_fractf(ang * 0.15915494309189535f);
  sn = __builtin_amdgcn_sinf(r);
  cn = __builtin_amdgcn_cosf(r);
}

// One token's raw inputs for one lane of a time loop: dt, lam, theta_k, the
// B (or C) pair of each rank (one packed word for bfloat16, two for float),
// the x (or dy) element of each rank.
template <typename T, int R>
struct StepIn {
  static constexpr int PW = sizeof(T) / 2;
  uint32_t d, l, th, v[R * PW], w[R];
};

template <typename T>
__device__ __forceinline__ void pair_of(const uint32_t* v, float& a0, float& a1) {
  if constexpr (sizeof(T) == 2) {
    a0 = __uint_as_float(v[0] << 16);
    a1 = __uint_as_float(v[0] & 0xffff0000u);
  } else {
    a0 = __uint_as_float(v[0]);
    a1 = __uint_as_float(v[1]);
  }
}
template <typename T>
__device__ __forceinline__ float elem_of(uint32_t w) {
  if constexpr (sizeof(T) == 2) return __uint_as_float(w << 16);
  else return __uint_as_float(w);
}

// Buffer ranges of one (batch, head) sequence: per-token rows start at the
// sequence's first token and advance by the token stride.
struct SeqRanges {
  brsrc dt, lam, th, pr, el;  // dt, lam, theta, B or C pairs, x or dy elements
  uint32_t sd, sth, spr, sel;  // token strides in bytes
};

template <typename T, int R>
__device__ __forceinline__ SeqRanges seq_ranges(const BackwardArgs& a, int b, int hh,
                                                const void* pairs, const void* elems) {
  constexpr uint32_t es = sizeof(T);
  const size_t tok0 = (size_t)b * a.T * a.H + hh;
  SeqRanges q;
  q.sd = (uint32_t)a.H * 4;
  q.sth = (uint32_t)a.H * (a.N / 2) * 4;
  q.spr = (uint32_t)a.H * R * a.N * es;
  q.sel = (uint32_t)a.H * R * a.P * es;
  const uint32_t last = (uint32_t)(a.T - 1);
  q.dt = mk_rsrc(a.dt + tok0, last * q.sd + 4);
  q.lam = mk_rsrc(a.lam + tok0, last * q.sd + 4);
  q.th = mk_rsrc(a.theta + tok0 * (a.N / 2), last * q.sth + (uint32_t)(a.N / 2) * 4);
  q.pr = mk_rsrc(static_cast<const unsigned char*>(pairs) + tok0 * R * a.N * es,
                 last * q.spr + (uint32_t)(R * a.N) * es);
  q.el = mk_rsrc(static_cast<const unsigned char*>(elems) + tok0 * R * a.P * es,
                 last * q.sel + (uint32_t)(R * a.P) * es);
  return q;
}

template <typename T, int R>
__device__ __forceinline__ void load_step(const SeqRanges& q, int t, int kp, int p, int N, int P,
                                          bool with_lam, StepIn<T, R>& in) {
  constexpr uint32_t es = sizeof(T);
  const uint32_t ut = (uint32_t)t;
  in.d = bld32(q.dt, ut * q.sd);
  in.l = with_lam ? bld32(q.lam, ut * q.sd) : 0u;
  in.th = bld32(q.th, ut * q.sth + (uint32_t)kp * 4);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t po = ut * q.spr + (uint32_t)(r * N + 2 * kp) * es;
    if constexpr (sizeof(T) == 2) {
      in.v[r] = bld32(q.pr, po);
      in.w[r] = bld16(q.el, ut * q.sel + (uint32_t)(r * P + p) * es);
    } else {
      in.v[2 * r] = bld32(q.pr, po);
      in.v[2 * r + 1] = bld32(q.pr, po + 4);
      in.w[r] = bld32(q.el, ut * q.sel + (uint32_t)(r * P + p) * es);
    }
  }
}

// One lane per (row pair kp, column p) of every (batch, head) unit.
template <typename T, int R>
__global__ void __launch_bounds__(kScanThreads) fwd_states_kernel(BackwardArgs a) {
  const int unit = blockIdx.x;  // b * H + h
  const int idx = blockIdx.y * kScanThreads + threadIdx.x;
  if (idx >= (a.N / 2) * a.P) return;
  const int kp = idx / a.P, p = idx % a.P;
  const int b = unit / a.H, hh = unit % a.H;
  const float Ah = a.A[hh];
  const size_t NP = (size_t)a.N * a.P;
  // the unit's states; stores past the last token fall outside the range
  const brsrc hs = mk_rsrc(a.hs + (size_t)unit * a.T * NP, (uint32_t)(a.T * NP * 4));
  const uint32_t lo = (uint32_t)((2 * kp) * a.P + p) * 4, sNP = (uint32_t)NP * 4;
  const SeqRanges q = seq_ranges<T, R>(a, b, hh, a.B, a.x);
  StepIn<T, R> ring[kAhead];
#pragma unroll
  for (int j = 0; j < kAhead; ++j) load_step<T, R>(q, j, kp, p, a.N, a.P, true, ring[j]);
  float h0 = 0.f, h1 = 0.f, q0 = 0.f, q1 = 0.f;  // state pair, previous P pair
  // whole groups of kAhead steps with no branch inside (a branch would copy
  // the staged values and wait for them); the steps past the last token
  // run on zeros and store nothing
  for (int t0 = 0; t0 < a.T; t0 += kAhead) {
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      const int t = t0 + j;
      const StepIn<T, R> in = ring[j];
      // unconditional: past the sequence's end the buffer range returns zeros
      load_step<T, R>(q, t + kAhead, kp, p, a.N, a.P, true, ring[j]);
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float b0, b1;
        pair_of<T>(in.v + r * StepIn<T, R>::PW, b0, b1);
        const float xv = elem_of<T>(in.w[r]);
        p0 = __builtin_fmaf(b0, xv, p0);
        p1 = __builtin_fmaf(b1, xv, p1);
      }
      const float d = __uint_as_float(in.d), l = __uint_as_float(in.l);
      const float alpha = __expf(d * Ah), beta = (1.f - l) * d, gamma = l * d;
      float sn, cn;
      sincos_step(d * __uint_as_float(in.th), sn, cn);
      const float u0 = __builtin_fmaf(beta, q0, h0), u1 = __builtin_fmaf(beta, q1, h1);
      h0 = __builtin_fmaf(alpha, cn * u0 - sn * u1, gamma * p0);
      h1 = __builtin_fmaf(alpha, sn * u0 + cn * u1, gamma * p1);
      bst32(h0, hs, (uint32_t)t * sNP + lo);
      bst32(h1, hs, (uint32_t)t * sNP + lo + (uint32_t)a.P * 4);
      q0 = p0;
      q1 = p1;
    }
  }
}

// G_t from t = T-1 down to 0, one lane per (row pair, column).
template <typename T, int R>
__global__ void __launch_bounds__(kScanThreads) adj_states_kernel(BackwardArgs a) {
  const int unit = blockIdx.x;
  const int idx = blockIdx.y * kScanThreads + threadIdx.x;
  if (idx >= (a.N / 2) * a.P) return;
  const int kp = idx / a.P, p = idx % a.P;
  const int b = unit / a.H, hh = unit % a.H;
  const float Ah = a.A[hh];
  const size_t NP = (size_t)a.N * a.P;
  const brsrc gs = mk_rsrc(a.gs + (size_t)unit * a.T * NP, (uint32_t)(a.T * NP * 4));
  const uint32_t lo = (uint32_t)((2 * kp) * a.P + p) * 4, sNP = (uint32_t)NP * 4;
  const SeqRanges q = seq_ranges<T, R>(a, b, hh, a.C, a.dy);
  // dU_{t+1}, starting with dh_final folded in at t = T-1
  float e0 = 0.f, e1 = 0.f;
  if (a.dh_final) {
    const float* df = a.dh_final + (size_t)unit * NP + (size_t)(2 * kp) * a.P + p;
    e0 = df[0];
    e1 = df[a.P];
  }
  // ring slot j holds token T-1-(s+j) at step s of the reversed walk
  StepIn<T, R> ring[kAhead];
#pragma unroll
  for (int j = 0; j < kAhead; ++j) load_step<T, R>(q, a.T - 1 - j, kp, p, a.N, a.P, false, ring[j]);
  // as in the forward loop: no branch inside a group; steps before the first
  // token run on zeros and their stores wrap past the range
  for (int s0 = 0; s0 < a.T; s0 += kAhead) {
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      const int sidx = s0 + j;
      const int t = a.T - 1 - sidx;
      const StepIn<T, R> in = ring[j];
      // unconditional: before the first token the offset wraps past the
      // buffer range and reads zeros
      load_step<T, R>(q, t - kAhead, kp, p, a.N, a.P, false, ring[j]);
      float g0 = e0, g1 = e1;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float c0, c1;
        pair_of<T>(in.v + r * StepIn<T, R>::PW, c0, c1);
        const float gv = elem_of<T>(in.w[r]);
        g0 = __builtin_fmaf(c0, gv, g0);
        g1 = __builtin_fmaf(c1, gv, g1);
      }
      bst32(g0, gs, (uint32_t)t * sNP + lo);
      bst32(g1, gs, (uint32_t)t * sNP + lo + (uint32_t)a.P * 4);
      // dU_t = alpha_t R_t^T G_t, the term G_{t-1} inherits
      const float d = __uint_as_float(in.d);
      const float alpha = __expf(d * Ah);
      float sn, cs;
      sincos_step(d * __uint_as_float(in.th), sn, cs);
      e0 = alpha * (cs * g0 + sn * g1);
      e1 = alpha * (cs * g1 - sn * g0);
    }
  }
}

// Sum over the `width` consecutive lanes of a group (width a power of two).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, width);
  return v;
}

// Eight consecutive elements (16 bytes of bfloat16, 32 of float) as float.
__device__ __forceinline__ void load8(const bf16* p, float (&v)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(ws[i] << 16);
    v[2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a0 = reinterpret_cast<const float4*>(p)[0], a1 = reinterpret_cast<const float4*>(p)[1];
  v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
  v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
}

constexpr int kTokPerBlock = 4;  // consecutive tokens of one sequence per workgroup

// One workgroup per kTokPerBlock consecutive tokens of one (batch, head);
// thread (kp, pc) holds rows 2kp, 2kp+1 and columns 8 pc .. 8 pc + 7 (pc
// fastest, so a row's threads are consecutive lanes and its loads coalesce).
// A token's h_t, B_t and x_t are the next token's h_{t-1}, B_{t-1}, x_{t-1}.
template <typename T, int R>
__global__ void __launch_bounds__(512) token_grads_kernel(BackwardArgs a) {
  extern __shared__ __align__(16) float bsm[];
  const int npc = a.P / 8;
  const int tid = threadIdx.x;
  const int kp = tid / npc, pc = tid % npc;
  const int nblk_t = (a.T + kTokPerBlock - 1) / kTokPerBlock;
  const size_t unit = blockIdx.x / nblk_t;  // b * H + h
  const int t0 = (int)(blockIdx.x % nblk_t) * kTokPerBlock;
  const int hh = (int)(unit % a.H);
  const size_t bidx = unit / a.H;
  const size_t NP = (size_t)a.N * a.P;
  const float Ah = a.A[hh];
  const T* xb = static_cast<const T*>(a.x);
  const T* Bb = static_cast<const T*>(a.B);
  const T* Cb = static_cast<const T*>(a.C);
  const T* dyb = static_cast<const T*>(a.dy);
  const size_t row0 = (size_t)(2 * kp) * a.P + 8 * pc;
  const float* hbase = a.hs + unit * a.T * NP + row0;
  const float* gbase = a.gs + unit * a.T * NP + row0;
  const int nkp = a.N / 2;
  float* s_dx = bsm;                           // [nkp][R * P]
  float* s_red = bsm + (size_t)nkp * R * a.P;  // [waves][4]
  const int ww = blockDim.x < 64 ? (int)blockDim.x : 64;
  const int lane = tid & 63, wave = tid >> 6, nw = (blockDim.x + 63) >> 6;

  // the previous token's state and inputs (zero before the first token)
  float hp[2][8], bq[R][2], xq[R][8];
  {
    const int tq = t0 - 1;
    const size_t tokq = (bidx * a.T + (tq < 0 ? 0 : tq)) * a.H + hh;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (tq >= 0) load8(hbase + (size_t)tq * NP + i * a.P, hp[i]);
      else
#pragma unroll
        for (int j = 0; j < 8; ++j) hp[i][j] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const size_t o = (tokq * R + r) * a.N + 2 * kp;
      bq[r][0] = tq >= 0 ? ldf(Bb + o) : 0.f;
      bq[r][1] = tq >= 0 ? ldf(Bb + o + 1) : 0.f;
      if (tq >= 0) load8(xb + (tokq * R + r) * a.P + 8 * pc, xq[r]);
      else
#pragma unroll
        for (int j = 0; j < 8; ++j) xq[r][j] = 0.f;
    }
  }

  for (int jt = 0; jt < kTokPerBlock; ++jt) {
    const int t = t0 + jt;
    if (t >= a.T) break;  // uniform over the block
    const size_t tok = (bidx * a.T + t) * a.H + hh;
    const float d = a.dt[tok], l = a.lam[tok];
    const float alpha = __expf(d * Ah), beta = (1.f - l) * d, gamma = l * d;
    const float beta_n = t + 1 < a.T ? (1.f - a.lam[tok + a.H]) * a.dt[tok + a.H] : 0.f;
    const float th = a.theta[tok * (a.N / 2) + kp];
    float sn, cn;
    sincos_step(d * th, sn, cn);
    float hc[2][8], gg[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      load8(hbase + (size_t)t * NP + i * a.P, hc[i]);
      load8(gbase + (size_t)t * NP + i * a.P, gg[i]);
    }
    float bc[R][2], cc[R][2], xc[R][8], dyc[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const size_t o = (tok * R + r) * a.N + 2 * kp;
      bc[r][0] = ldf(Bb + o); bc[r][1] = ldf(Bb + o + 1);
      cc[r][0] = ldf(Cb + o); cc[r][1] = ldf(Cb + o + 1);
      load8(xb + (tok * R + r) * a.P + 8 * pc, xc[r]);
      load8(dyb + (tok * R + r) * a.P + 8 * pc, dyc[r]);
    }
    float s_alpha = 0.f, s_gamma = 0.f, s_beta = 0.f, s_psi = 0.f;
    float dBp[R][2], dCp[R][2], dxp[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      dBp[r][0] = dBp[r][1] = dCp[r][0] = dCp[r][1] = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) dxp[r][j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float pc0 = 0.f, pc1 = 0.f, pq0 = 0.f, pq1 = 0.f, cd0 = 0.f, cd1 = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        pc0 = __builtin_fmaf(bc[r][0], xc[r][j], pc0);
        pc1 = __builtin_fmaf(bc[r][1], xc[r][j], pc1);
        pq0 = __builtin_fmaf(bq[r][0], xq[r][j], pq0);
        pq1 = __builtin_fmaf(bq[r][1], xq[r][j], pq1);
        cd0 = __builtin_fmaf(cc[r][0], dyc[r][j], cd0);
        cd1 = __builtin_fmaf(cc[r][1], dyc[r][j], cd1);
      }
      const float g0 = gg[0][j], g1 = gg[1][j];
      const float u0 = __builtin_fmaf(beta, pq0, hp[0][j]), u1 = __builtin_fmaf(beta, pq1, hp[1][j]);
      const float v0 = cn * u0 - sn * u1, v1 = sn * u0 + cn * u1;  // R U
      s_alpha += g0 * v0 + g1 * v1;
      s_psi += g1 * v0 - g0 * v1;  // <G, R'(psi) U>
      const float du0 = alpha * (cn * g0 + sn * g1), du1 = alpha * (cn * g1 - sn * g0);  // dU_t
      s_gamma += g0 * pc0 + g1 * pc1;
      s_beta += du0 * pq0 + du1 * pq1;
      // dU_{t+1} = G_t - C dy^T (zero past the last token)
      const float un0 = t + 1 < a.T ? g0 - cd0 : 0.f, un1 = t + 1 < a.T ? g1 - cd1 : 0.f;
      const float dp0 = __builtin_fmaf(beta_n, un0, gamma * g0);
      const float dp1 = __builtin_fmaf(beta_n, un1, gamma * g1);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        dBp[r][0] = __builtin_fmaf(dp0, xc[r][j], dBp[r][0]);
        dBp[r][1] = __builtin_fmaf(dp1, xc[r][j], dBp[r][1]);
        dCp[r][0] = __builtin_fmaf(hc[0][j], dyc[r][j], dCp[r][0]);
        dCp[r][1] = __builtin_fmaf(hc[1][j], dyc[r][j], dCp[r][1]);
        dxp[r][j] = dp0 * bc[r][0] + dp1 * bc[r][1];
      }
    }
    // sums over the columns: the row pair's npc consecutive lanes
    s_psi = group_sum(s_psi, npc);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      dBp[r][0] = group_sum(dBp[r][0], npc);
      dBp[r][1] = group_sum(dBp[r][1], npc);
      dCp[r][0] = group_sum(dCp[r][0], npc);
      dCp[r][1] = group_sum(dCp[r][1], npc);
    }
    if (pc == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const size_t o = (tok * R + r) * a.N + 2 * kp;
        a.dB[o] = dBp[r][0];
        a.dB[o + 1] = dBp[r][1];
        a.dC[o] = dCp[r][0];
        a.dC[o + 1] = dCp[r][1];
      }
      a.dtheta[tok * (a.N / 2) + kp] = alpha * s_psi * d;
    }
    // dx: sums over the row pairs through LDS, a fixed order
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j) s_dx[(size_t)kp * R * a.P + r * a.P + 8 * pc + j] = dxp[r][j];
    // scalars (the theta terms of d dt once per row pair)
    float sv[4] = {s_alpha, s_gamma, s_beta, pc == 0 ? alpha * s_psi * th : 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      for (int off = ww >> 1; off > 0; off >>= 1) sv[q] += __shfl_xor(sv[q], off, ww);
      if (lane == 0) s_red[wave * 4 + q] = sv[q];
    }
    __syncthreads();
    for (int o = tid; o < R * a.P; o += blockDim.x) {
      float sum = 0.f;
      for (int k = 0; k < nkp; ++k) sum += s_dx[(size_t)k * R * a.P + o];
      a.dx[tok * R * a.P + o] = sum;
    }
    if (tid == 0) {
      float tot[4] = {0.f, 0.f, 0.f, 0.f};
      for (int w = 0; w < nw; ++w)
#pragma unroll
        for (int q = 0; q < 4; ++q) tot[q] += s_red[w * 4 + q];
      const float dal = tot[0], dga = tot[1], dbe = tot[2];
      a.ddt[tok] = dal * alpha * Ah + dbe * (1.f - l) + dga * l + tot[3];
      a.dlam[tok] = (dga - dbe) * d;
      a.dAc[tok] = dal * alpha * d;
    }
    __syncthreads();  // s_dx and s_red are rewritten by the next token
    // this token is the next one's previous token
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) hp[i][j] = hc[i][j];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      bq[r][0] = bc[r][0];
      bq[r][1] = bc[r][1];
#pragma unroll
      for (int j = 0; j < 8; ++j) xq[r][j] = xc[r][j];
    }
  }
}

__global__ void zero_kernel(float* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// dA[h] = sum over (batch, time) of the per-token contributions, in a fixed
// order: each thread a strided partial sum, then a tree over the block.
__global__ void __launch_bounds__(256) dA_kernel(BackwardArgs a) {
  __shared__ float s[256];
  const int hh = blockIdx.x;
  const size_t n = (size_t)a.nb * a.T;
  float v = 0.f;
  for (size_t i = threadIdx.x; i < n; i += 256) v += a.dAc[i * a.H + hh];
  s[threadIdx.x] = v;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) s[threadIdx.x] += s[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.dA[hh] = s[0];
}

template <typename T, int R>
hipError_t launch_typed(const BackwardArgs& a, hipStream_t stream) {
  const int units = a.nb * a.H;
  const dim3 sgrid(units, (unsigned)(((a.N / 2) * a.P + kScanThreads - 1) / kScanThreads));
  hipLaunchKernelGGL((fwd_states_kernel<T, R>), sgrid, dim3(kScanThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((adj_states_kernel<T, R>), sgrid, dim3(kScanThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int threads = (a.N / 2) * (a.P / 8);
  const size_t lds = sizeof(float) * ((size_t)(a.N / 2) * R * a.P + 4 * ((threads + 63) / 64));
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&token_grads_kernel<T, R>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const size_t nblk_t = ((size_t)a.T + kTokPerBlock - 1) / kTokPerBlock;
  hipLaunchKernelGGL((token_grads_kernel<T, R>), dim3((unsigned)((size_t)a.nb * a.H * nblk_t)),
                     dim3(threads), lds, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dA_kernel, dim3(a.H), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const BackwardArgs& a, hipStream_t stream) {
  switch (a.R) {
    case 1: return launch_typed<T, 1>(a, stream);
    case 2: return launch_typed<T, 2>(a, stream);
    case 4: return launch_typed<T, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, m3_dtype dtype, hipStream_t stream) {
  if (a.nb == 0 || a.T == 0) {
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((a.H + 255) / 256)), dim3(256), 0, stream,
                       a.dA, a.H);
    return hipGetLastError();
  }
  return dtype == M3_BF16 ? launch_t<bf16>(a, stream) : launch_t<float>(a, stream);
}

}  // namespace m3
