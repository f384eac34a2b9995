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
// loop each way, the next token's inputs prefetched); token_grads_kernel
// then forms every token's gradients in parallel from h_t, h_{t-1} and G_t
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
  float* hs = a.hs + (size_t)unit * a.T * NP + (size_t)(2 * kp) * a.P + p;
  const T* xb = static_cast<const T*>(a.x);
  const T* Bb = static_cast<const T*>(a.B);
  float h0 = 0.f, h1 = 0.f, q0 = 0.f, q1 = 0.f;  // state pair, previous P pair
  // inputs of token t (tok = (b*T + t)*H + hh)
  auto load = [&](int t, float& d, float& l, float& th, float (&bv)[2 * R], float (&xv)[R]) {
    const size_t tok = ((size_t)b * a.T + t) * a.H + hh;
    d = a.dt[tok];
    l = a.lam[tok];
    th = a.theta[tok * (a.N / 2) + kp];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      bv[2 * r] = ldf(Bb + (tok * R + r) * a.N + 2 * kp);
      bv[2 * r + 1] = ldf(Bb + (tok * R + r) * a.N + 2 * kp + 1);
      xv[r] = ldf(xb + (tok * R + r) * a.P + p);
    }
  };
  float d, l, th, bv[2 * R], xv[R];
  load(0, d, l, th, bv, xv);
  for (int t = 0; t < a.T; ++t) {
    float dn = 0.f, ln = 0.f, thn = 0.f, bn[2 * R], xn[R];
    if (t + 1 < a.T) load(t + 1, dn, ln, thn, bn, xn);
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      p0 = __builtin_fmaf(bv[2 * r], xv[r], p0);
      p1 = __builtin_fmaf(bv[2 * r + 1], xv[r], p1);
    }
    const float alpha = __expf(d * Ah), beta = (1.f - l) * d, gamma = l * d;
    float sn, cn;
    sincosf(d * th, &sn, &cn);
    const float u0 = __builtin_fmaf(beta, q0, h0), u1 = __builtin_fmaf(beta, q1, h1);
    h0 = __builtin_fmaf(alpha, cn * u0 - sn * u1, gamma * p0);
    h1 = __builtin_fmaf(alpha, sn * u0 + cn * u1, gamma * p1);
    hs[(size_t)t * NP] = h0;
    hs[(size_t)t * NP + a.P] = h1;
    q0 = p0;
    q1 = p1;
    if (t + 1 < a.T) {
      d = dn; l = ln; th = thn;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        bv[2 * r] = bn[2 * r]; bv[2 * r + 1] = bn[2 * r + 1]; xv[r] = xn[r];
      }
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
  float* gs = a.gs + (size_t)unit * a.T * NP + (size_t)(2 * kp) * a.P + p;
  const T* Cb = static_cast<const T*>(a.C);
  const T* dyb = static_cast<const T*>(a.dy);
  // dU_{t+1}, starting with dh_final folded in at t = T-1
  float e0 = 0.f, e1 = 0.f;
  if (a.dh_final) {
    const float* df = a.dh_final + (size_t)unit * NP + (size_t)(2 * kp) * a.P + p;
    e0 = df[0];
    e1 = df[a.P];
  }
  auto load = [&](int t, float& d, float& th, float (&cv)[2 * R], float (&gv)[R]) {
    const size_t tok = ((size_t)b * a.T + t) * a.H + hh;
    d = a.dt[tok];
    th = a.theta[tok * (a.N / 2) + kp];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      cv[2 * r] = ldf(Cb + (tok * R + r) * a.N + 2 * kp);
      cv[2 * r + 1] = ldf(Cb + (tok * R + r) * a.N + 2 * kp + 1);
      gv[r] = ldf(dyb + (tok * R + r) * a.P + p);
    }
  };
  float d, th, cv[2 * R], gv[R];
  load(a.T - 1, d, th, cv, gv);
  for (int t = a.T - 1; t >= 0; --t) {
    float dn = 0.f, thn = 0.f, cn_[2 * R], gn[R];
    if (t > 0) load(t - 1, dn, thn, cn_, gn);
    float g0 = e0, g1 = e1;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      g0 = __builtin_fmaf(cv[2 * r], gv[r], g0);
      g1 = __builtin_fmaf(cv[2 * r + 1], gv[r], g1);
    }
    gs[(size_t)t * NP] = g0;
    gs[(size_t)t * NP + a.P] = g1;
    // dU_t = alpha_t R_t^T G_t, the term G_{t-1} inherits
    const float alpha = __expf(d * Ah);
    float sn, cs;
    sincosf(d * th, &sn, &cs);
    e0 = alpha * (cs * g0 + sn * g1);
    e1 = alpha * (cs * g1 - sn * g0);
    if (t > 0) {
      d = dn; th = thn;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        cv[2 * r] = cn_[2 * r]; cv[2 * r + 1] = cn_[2 * r + 1]; gv[r] = gn[r];
      }
    }
  }
}

// Sum over the `width` consecutive lanes of a group (width a power of two).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, width);
  return v;
}

// One workgroup per token-head; thread (kp, pc) holds rows 2kp, 2kp+1 and
// columns 8 pc .. 8 pc + 7 (pc fastest, so a row's eight threads are
// consecutive lanes and its loads coalesce).
template <typename T, int R>
__global__ void __launch_bounds__(512) token_grads_kernel(BackwardArgs a) {
  extern __shared__ __align__(16) float bsm[];
  const int npc = a.P / 8;
  const int tid = threadIdx.x;
  const int kp = tid / npc, pc = tid % npc;
  const size_t th_id = blockIdx.x;  // (b * T + t) * H + h
  const int hh = (int)(th_id % a.H);
  const size_t bt = th_id / a.H;
  const int t = (int)(bt % a.T);
  const size_t unit = (bt / a.T) * a.H + hh;
  const size_t NP = (size_t)a.N * a.P;
  const size_t tok = th_id;
  const float Ah = a.A[hh];
  const float d = a.dt[tok], l = a.lam[tok];
  const float alpha = __expf(d * Ah), beta = (1.f - l) * d, gamma = l * d;
  const float beta_n = t + 1 < a.T ? (1.f - a.lam[tok + a.H]) * a.dt[tok + a.H] : 0.f;
  const float th = a.theta[tok * (a.N / 2) + kp];
  float sn, cn;
  sincosf(d * th, &sn, &cn);
  const T* xb = static_cast<const T*>(a.x);
  const T* Bb = static_cast<const T*>(a.B);
  const T* Cb = static_cast<const T*>(a.C);
  const T* dyb = static_cast<const T*>(a.dy);
  const size_t row0 = (size_t)(2 * kp) * a.P + 8 * pc;
  const float* hcur = a.hs + (unit * a.T + t) * NP + row0;
  const float* gcur = a.gs + (unit * a.T + t) * NP + row0;
  float hc[2][8], hp[2][8], gg[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      hc[i][j] = hcur[i * a.P + j];
      gg[i][j] = gcur[i * a.P + j];
      hp[i][j] = t > 0 ? hcur[i * a.P + j - NP] : 0.f;
    }
  // token inputs: B, C pairs of this row pair; x, dy columns of this group
  float bc[R][2], bq[R][2], cc[R][2], xc[R][8], xq[R][8], dyc[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const size_t o = (tok * R + r) * a.N + 2 * kp;
    bc[r][0] = ldf(Bb + o); bc[r][1] = ldf(Bb + o + 1);
    cc[r][0] = ldf(Cb + o); cc[r][1] = ldf(Cb + o + 1);
    const size_t oq = o - (size_t)a.H * R * a.N;  // previous token of the sequence
    bq[r][0] = t > 0 ? ldf(Bb + oq) : 0.f;
    bq[r][1] = t > 0 ? ldf(Bb + oq + 1) : 0.f;
    const size_t ox = (tok * R + r) * a.P + 8 * pc;
    const size_t oxq = ox - (size_t)a.H * R * a.P;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      xc[r][j] = ldf(xb + ox + j);
      xq[r][j] = t > 0 ? ldf(xb + oxq + j) : 0.f;
      dyc[r][j] = ldf(dyb + ox + j);
    }
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
    s_psi += g1 * v0 - g0 * v1;  // <G, R'(psi) U> / 1
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
  const int nkp = a.N / 2;
  float* s_dx = bsm;                         // [nkp][R * P]
  float* s_red = bsm + (size_t)nkp * R * a.P;  // [waves][4]
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < 8; ++j) s_dx[(size_t)kp * R * a.P + r * a.P + 8 * pc + j] = dxp[r][j];
  // scalars: per-thread psi terms enter d dt through theta
  float s_dt_psi = alpha * s_psi * th;  // one value per row pair (lane pc = 0 after the sum)
  if (pc != 0) s_dt_psi = 0.f;
  float sv[4] = {s_alpha, s_gamma, s_beta, s_dt_psi};
  // blockDim is a power of two (16 .. 512): a block smaller than a wave
  // reduces over its own lanes only
  const int ww = blockDim.x < 64 ? (int)blockDim.x : 64;
  const int lane = tid & 63, wave = tid >> 6, nw = (blockDim.x + 63) >> 6;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    for (int off = ww >> 1; off > 0; off >>= 1) sv[q] += __shfl_xor(sv[q], off, ww);
    if (lane == 0) s_red[wave * 4 + q] = sv[q];
  }
  __syncthreads();
  for (int o = tid; o < R * a.P; o += blockDim.x) {
    float s = 0.f;
    for (int k = 0; k < nkp; ++k) s += s_dx[(size_t)k * R * a.P + o];
    a.dx[tok * R * a.P + o] = s;
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
  hipLaunchKernelGGL((token_grads_kernel<T, R>), dim3((unsigned)((size_t)a.nb * a.T * a.H)),
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
