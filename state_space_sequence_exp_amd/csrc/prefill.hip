// prefill.hip -- chunked prefill of the Mamba-3 recurrence on gfx950.
//
// Three kernels per call, all on the caller's stream:
//
//  1. chunk_state  (one block per (b, h, chunk)): per-token log-decay prefix
//     sums cs_u (wave scan), trapezoid weights gamma_u = lam_u dt_u and
//     omega_u = (1 - lam_{u+1}) dt_{u+1}, chunk-local cumulative angles
//     phi_u[k] = sum dt theta (segmented scan over tokens), the rotated inputs
//     B~_u = R(phi_u)^T B_u (the data-dependent RoPE of Proposition 3, Mamba-3
//     paper summary), and the chunk-local state
//         S_c = sum_u exp(cs_e - cs_u) (gamma_u + omega_u) B~_u x_u^T
//     as an MFMA contraction over the chunk's L*R (token, rank) rows.
//  2. state_scan   (elementwise over (b, h, p, pair)): the chunk-level
//     recurrence G_{c+1} = R(Phi_c) (exp(cs_e) G_c + S_c), G_0 = 0, storing
//     every chunk's entry state G_c and the final state.
//  3. chunk_out    (one block per (b, h, chunk)): rotated B~, C~ again and
//         y_t = exp(cs_t) C~_t^T G_c
//             + sum_{u<=t} exp(cs_t - cs_u)(gamma_u + [u<t] omega_u) (C~_t^T B~_u) x_u^T
//     i.e. the chunk's structured mask (decay matrix x 2-band trapezoid
//     matrix; Mamba-3 paper translation, section 3.1, equation 7) applied to
//     C~ B~^T, on MFMA, plus the inter-chunk term from the entry state.
//
// Frames.  Angles restart at every chunk, so the entry state G_c of a chunk
// is in the unrotated (API) frame, and the previous token's trapezoid term
// omega B x^T is folded into G_c: G_c = h_{cL-1} + omega_{cL-1} B_{cL-1}
// x_{cL-1}^T.  This needs no halo token inside a chunk and keeps every angle
// bounded by one chunk's sum.  The chunk-level recurrence (explainer,
// yunpan.plus: parallel inside a chunk, recurrent across chunks) then only
// needs each chunk's total decay and total angle.
//
// Layouts in LDS put the contraction dimension contiguous for both MFMA
// operands: C~, B~ as [row][N]; X^T and (B~ coef)^T as [col][row].  Chunk
// states are stored [P][N] so that rotation pairs are adjacent and the
// entry state is directly an MFMA B operand.
#include "m3_device.h"
#include "m3_internal.h"

namespace m3 {
namespace {

struct Chunk {
  int b, h, c, t0, len;
  size_t bh;
};

__device__ __forceinline__ Chunk chunk_of_block(const PrefillArgs& a) {
  Chunk k;
  const int blk = blockIdx.x;
  k.c = blk % a.nC;
  const int bh = blk / a.nC;
  k.bh = (size_t)bh;
  k.b = bh / a.H;
  k.h = bh % a.H;
  k.t0 = k.c * a.L;
  k.len = min(a.L, a.T - k.t0);
  return k;
}

// Per-token scalars of the chunk into LDS: cs (inclusive prefix of dt*A),
// gamma, omega and dt; padded tokens (u >= len) get zeros.
__device__ void load_scalars(const PrefillArgs& a, const Chunk& k, float* s_cs, float* s_gam,
                             float* s_om, float* s_dt) {
  const int tid = threadIdx.x;
  if (tid < 2 * kWave) {
    const int u = tid;
    float d = 0.f, la = 0.f, om = 0.f;
    if (u < k.len) {
      const size_t i = ((size_t)k.b * a.T + k.t0 + u) * a.H + k.h;
      d = a.dt[i];
      la = a.lam[i];
      if (k.t0 + u + 1 < a.T) {
        const size_t i1 = i + a.H;
        om = (1.f - a.lam[i1]) * a.dt[i1];
      }
    }
    const float cs = wave_incl_scan(d * a.A[k.h]);
    if (u < kLMax) {
      s_cs[u] = cs;
      s_gam[u] = la * d;
      s_om[u] = om;
      s_dt[u] = d;
    }
  }
  __syncthreads();
  if (tid >= kWave && tid < 2 * kWave) s_cs[tid] += s_cs[kWave - 1];
  __syncthreads();
}

// X^T tile: sXT[p][row] = x[token row/R][rank row%R][p], zero outside the chunk.
template <typename T>
__device__ void load_xT(const PrefillArgs& a, const Chunk& k, const ChunkLayout& lay, T* sXT) {
  constexpr int vec = 16 / sizeof(T);
  const int tpr = a.P / vec;
  const int rows_per_pass = kThreads / tpr;
  const int tid = threadIdx.x;
  const int p0 = (tid % tpr) * vec;
  const T* x = static_cast<const T*>(a.x);
  for (int row = tid / tpr; row < lay.LRpad; row += rows_per_pass) {
    const int u = row / a.R, r = row % a.R;
    T v[vec];
    if (row < lay.LR && u < k.len) {
      const size_t off = ((((size_t)k.b * a.T + k.t0 + u) * a.H + k.h) * a.R + r) * a.P + p0;
      const uint4 raw = *reinterpret_cast<const uint4*>(x + off);
      const T* rv = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int e = 0; e < vec; ++e) v[e] = rv[e];
    } else {
#pragma unroll
      for (int e = 0; e < vec; ++e) v[e] = from_f32<T>(0.f);
    }
#pragma unroll
    for (int e = 0; e < vec; ++e) sXT[(p0 + e) * lay.ldK + row] = v[e];
  }
}

// Chunk-local cumulative angles and rotated inputs.
//   kOut = false: writes (B~ * coef)^T into sA ([N][ldK]) and the chunk's
//                 (cos, sin) of the total angle to a.rot.
//   kOut = true : writes C~ into sA and B~ into sB (both [LRpad][ldN]).
template <typename T, bool kOut>
__device__ void rotate_inputs(const PrefillArgs& a, const Chunk& k, const ChunkLayout& lay,
                              const float* s_cs, const float* s_gam, const float* s_om,
                              const float* s_dt, float* s_part, T* sA, T* sB) {
  const int tid = threadIdx.x;
  const int npair = a.N / 2;
  const int nseg = kThreads / npair;
  const int kp = tid % npair, seg = tid / npair;
  const bool active = seg < nseg;
  const int seglen = (a.L + nseg - 1) / nseg;
  const int u0 = seg * seglen, u1 = min(a.L, u0 + seglen);
  const size_t tok_stride_th = (size_t)a.H * npair;
  const float* th = a.theta + (((size_t)k.b * a.T + k.t0) * a.H + k.h) * npair + kp;
  const int lenu = min(u1, k.len);

  RevSum sum;
  if (active)
    for (int u = u0; u < lenu; ++u) sum.add_rad(s_dt[u] * th[u * tok_stride_th]);
  if (active) {
    s_part[seg * npair + kp] = sum.hi;
    s_part[(nseg + seg) * npair + kp] = sum.lo;
  }

  // zero the padding rows [LR, LRpad)
  if (kOut) {
    for (int i = tid; i < (lay.LRpad - lay.LR) * a.N; i += kThreads) {
      const int row = lay.LR + i / a.N, n = i % a.N;
      sA[row * lay.ldN + n] = from_f32<T>(0.f);
      sB[row * lay.ldN + n] = from_f32<T>(0.f);
    }
  } else {
    for (int i = tid; i < (lay.LRpad - lay.LR) * a.N; i += kThreads) {
      const int col = lay.LR + i % (lay.LRpad - lay.LR), n = i / (lay.LRpad - lay.LR);
      sA[n * lay.ldK + col] = from_f32<T>(0.f);
    }
  }
  __syncthreads();
  if (!active) return;

  RevSum pre;
  for (int s = 0; s < seg; ++s) pre.add(s_part[s * npair + kp], s_part[(nseg + s) * npair + kp]);
  float phi = pre.radians();
  const float cs_end = s_cs[a.L - 1];
  const T* Bg = static_cast<const T*>(a.B);
  const T* Cg = static_cast<const T*>(a.C);
  const size_t tok_stride_bn = (size_t)a.H * a.R * a.N;
  const size_t base_bn = (((size_t)k.b * a.T + k.t0) * a.H + k.h) * a.R * a.N + 2 * kp;
  for (int u = u0; u < u1; ++u) {
    float sn = 0.f, cn = 1.f, coef = 0.f;
    const bool real = u < k.len;
    if (real) {
      phi = angle_add(phi, s_dt[u] * th[u * tok_stride_th]);
      fast_sincos(phi, &sn, &cn);
      if (!kOut) coef = __expf(cs_end - s_cs[u]) * (s_gam[u] + s_om[u]);
    }
    for (int r = 0; r < a.R; ++r) {
      const int row = u * a.R + r;
      float2 bv = make_float2(0.f, 0.f), cv = make_float2(0.f, 0.f);
      if (real) {
        const size_t off = base_bn + u * tok_stride_bn + (size_t)r * a.N;
        bv = load_pair(Bg + off);
        if (kOut) cv = load_pair(Cg + off);
      }
      // R(phi)^T applied to the pair
      const float b0 = cn * bv.x + sn * bv.y, b1 = -sn * bv.x + cn * bv.y;
      if (kOut) {
        const float c0 = cn * cv.x + sn * cv.y, c1 = -sn * cv.x + cn * cv.y;
        sA[row * lay.ldN + 2 * kp] = from_f32<T>(c0);
        sA[row * lay.ldN + 2 * kp + 1] = from_f32<T>(c1);
        sB[row * lay.ldN + 2 * kp] = from_f32<T>(b0);
        sB[row * lay.ldN + 2 * kp + 1] = from_f32<T>(b1);
      } else {
        sA[(2 * kp) * lay.ldK + row] = from_f32<T>(b0 * coef);
        sA[(2 * kp + 1) * lay.ldK + row] = from_f32<T>(b1 * coef);
      }
    }
  }
  if (!kOut && u1 == a.L && u0 < a.L) {
    // The scan chains this rotation over every chunk, so its angle is the
    // exact sum of the segment sums and its sine/cosine the accurate ones.
    pre.add(s_part[seg * npair + kp], s_part[(nseg + seg) * npair + kp]);
    float sn, cn;
    sincospif(2.f * pre.revolutions(), &sn, &cn);
    a.rot[(k.bh * a.nC + k.c) * npair + kp] = make_float2(cn, sn);
  }
}

// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(kThreads) chunk_state_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Chunk k = chunk_of_block(a);
  const ChunkLayout lay = chunk_layout(a.L, a.R, a.N, a.P, sizeof(T), false);
  float* s_cs = reinterpret_cast<float*>(smem + lay.off_scal);
  float* s_gam = s_cs + kLMax;
  float* s_om = s_gam + kLMax;
  float* s_dt = s_om + kLMax;
  float* s_part = reinterpret_cast<float*>(smem + lay.off_part);
  T* sBcT = reinterpret_cast<T*>(smem + lay.off_a);
  T* sXT = reinterpret_cast<T*>(smem + lay.off_xt);

  load_scalars(a, k, s_cs, s_gam, s_om, s_dt);
  load_xT<T>(a, k, lay, sXT);
  rotate_inputs<T, false>(a, k, lay, s_cs, s_gam, s_om, s_dt, s_part, sBcT, nullptr);
  if (threadIdx.x == 0) a.decay[k.bh * a.nC + k.c] = __expf(s_cs[a.L - 1]);
  __syncthreads();

  using M = Mfma<T>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int ntp = a.P / 16, ntn = a.N / 16;
  float* Sc = a.S + (k.bh * a.nC + k.c) * (size_t)a.P * a.N;
  for (int tile = wave; tile < ntp * ntn; tile += kThreads / kWave) {
    const int pt = tile / ntn, nt = tile % ntn;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < lay.LRpad; k0 += M::K) {
      const typename M::frag fa = M::load(sXT, lay.ldK, pt * 16 + li, k0);
      const typename M::frag fb = M::load(sBcT, lay.ldK, nt * 16 + li, k0);
      acc = M::mma(fa, fb, acc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) Sc[(size_t)(pt * 16 + 4 * g + j) * a.N + nt * 16 + li] = acc[j];
  }
}

// ---------------------------------------------------------------------------
// One thread per (b*h, p, pair); sequential over chunks.
template <typename T>
__global__ void __launch_bounds__(kThreads) state_scan_kernel(PrefillArgs a) {
  const int npair = a.N / 2;
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= a.P * npair) return;
  const size_t bh = blockIdx.y;
  const int p = idx / npair, kp = idx % npair;
  T* G = static_cast<T*>(a.G);
  float sx = 0.f, sy = 0.f;
  size_t off = (bh * a.nC * a.P + p) * a.N + 2 * kp;
  const size_t cstride = (size_t)a.P * a.N;
  for (int c = 0; c < a.nC; ++c, off += cstride) {
    G[off] = from_f32<T>(sx);
    G[off + 1] = from_f32<T>(sy);
    const float2 s = *reinterpret_cast<const float2*>(a.S + off);
    const float d = a.decay[bh * a.nC + c];
    const float2 rc = a.rot[(bh * a.nC + c) * npair + kp];
    const float vx = d * sx + s.x, vy = d * sy + s.y;
    sx = rc.x * vx - rc.y * vy;
    sy = rc.y * vx + rc.x * vy;
  }
  if (a.h_final) {
    a.h_final[(bh * a.N + 2 * kp) * a.P + p] = sx;
    a.h_final[(bh * a.N + 2 * kp + 1) * a.P + p] = sy;
  }
}

// ---------------------------------------------------------------------------
template <typename T, int P>
__global__ void __launch_bounds__(kThreads) chunk_out_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Chunk k = chunk_of_block(a);
  const ChunkLayout lay = chunk_layout(a.L, a.R, a.N, P, sizeof(T), true);
  float* s_cs = reinterpret_cast<float*>(smem + lay.off_scal);
  float* s_gam = s_cs + kLMax;
  float* s_om = s_gam + kLMax;
  float* s_dt = s_om + kLMax;
  float* s_part = reinterpret_cast<float*>(smem + lay.off_part);
  T* sC = reinterpret_cast<T*>(smem + lay.off_a);
  T* sB = reinterpret_cast<T*>(smem + lay.off_b);
  T* sXT = reinterpret_cast<T*>(smem + lay.off_xt);

  load_scalars(a, k, s_cs, s_gam, s_om, s_dt);
  load_xT<T>(a, k, lay, sXT);
  rotate_inputs<T, true>(a, k, lay, s_cs, s_gam, s_om, s_dt, s_part, sC, sB);
  __syncthreads();

  using M = Mfma<T>;
  constexpr int NPT = P / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int R = a.R, N = a.N;
  const T* Gc = static_cast<const T*>(a.G) + (k.bh * a.nC + k.c) * (size_t)P * N;
  T* y = static_cast<T*>(a.y);
  const int nqb = lay.LR / 16;

  for (int qb = wave; qb < nqb; qb += kThreads / kWave) {
    f32x4 acc[NPT];
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // inter-chunk term: C~ G_c, rows scaled by exp(cs_t)
    for (int n0 = 0; n0 < N; n0 += M::K) {
      const typename M::frag fa = M::load(sC, lay.ldN, qb * 16 + li, n0);
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        const typename M::frag fb = M::load(Gc, N, pt * 16 + li, n0);
        acc[pt] = M::mma(fa, fb, acc[pt]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sc = __expf(s_cs[(qb * 16 + 4 * g + j) / R]);
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) acc[pt][j] *= sc;
    }

    // intra-chunk term: (C~ B~^T o W) X over key blocks up to the diagonal
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
      // structured mask: decay x 2-band trapezoid weights
#pragma unroll
      for (int i = 0; i < KB; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tk = ((kb + i) * 16 + 4 * g + j) / R;
          float w = 0.f;
          if (tk < tq)
            w = __expf(csq - s_cs[tk]) * (s_gam[tk] + s_om[tk]);
          else if (tk == tq)
            w = s_gam[tk];
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
        for (int pt = 0; pt < NPT; ++pt) {
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
        for (int pt = 0; pt < NPT; ++pt) {
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
      const int u = row / R, r = row % R;
      if (u < k.len) {
        const size_t off = ((((size_t)k.b * a.T + k.t0 + u) * a.H + k.h) * R + r) * P + li;
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) y[off + pt * 16] = from_f32<T>(acc[pt][j]);
      }
    }
  }
}

template <typename T, int P>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream) {
  const int nblk = a.nb * a.H * a.nC;
  const ChunkLayout ls = chunk_layout(a.L, a.R, a.N, a.P, sizeof(T), false);
  const ChunkLayout lo = chunk_layout(a.L, a.R, a.N, a.P, sizeof(T), true);
  hipError_t e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_state_kernel<T>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)ls.total);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_out_kernel<T, P>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lo.total);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chunk_state_kernel<T>, dim3(nblk), dim3(kThreads), ls.total, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int per_bh = a.P * (a.N / 2);
  hipLaunchKernelGGL(state_scan_kernel<T>, dim3((per_bh + kThreads - 1) / kThreads, a.nb * a.H),
                     dim3(kThreads), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((chunk_out_kernel<T, P>), dim3(nblk), dim3(kThreads), lo.total, stream, a);
  return hipGetLastError();
}

__global__ void fill_zero_kernel(float* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, m3_dtype dtype, hipStream_t stream) {
  if (a.nb == 0) return hipSuccess;
  if (a.T == 0) {
    if (!a.h_final) return hipSuccess;
    const size_t n = (size_t)a.nb * a.H * a.N * a.P;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       a.h_final, n);
    return hipGetLastError();
  }
  const bool bf = dtype == M3_BF16;
  switch (a.P) {
    case 16: return bf ? launch_typed<bf16, 16>(a, stream) : launch_typed<float, 16>(a, stream);
    case 32: return bf ? launch_typed<bf16, 32>(a, stream) : launch_typed<float, 32>(a, stream);
    case 64: return bf ? launch_typed<bf16, 64>(a, stream) : launch_typed<float, 64>(a, stream);
    case 128: return bf ? launch_typed<bf16, 128>(a, stream) : launch_typed<float, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace m3
