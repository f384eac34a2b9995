// m3ssm_api.hip -- the C ABI of libm3ssm (declared in include/m3ssm.h):
// argument validation, workspace carving and kernel dispatch.  Everything is
// checked on the host before any HIP call, so an invalid call enqueues
// nothing.
#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "m3_internal.h"
#include "m3ssm.h"

// Scratch of m3_prefill_noalloc (see device_scratch below): one copy per GPU.
static __device__ __align__(256) unsigned char scratch[M3_PREFILL_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

bool valid_p(int64_t P) { return P == 16 || P == 32 || P == 64 || P == 128; }
bool valid_r(int64_t R) { return R == 1 || R == 2 || R == 4; }

size_t esize_of(m3_dtype d) { return d == M3_BF16 ? 2 : 4; }

// The C callers may pass any int for an enum parameter; in C++ reading an
// enum object that holds a value outside its enumerators' range is undefined,
// so the public entry points first read the object's bytes as an int.
int enum_bits(const void* e) {
  int v;
  memcpy(&v, e, sizeof v);
  return v;
}
bool dtype_ok(const m3_dtype* d) {
  const int v = enum_bits(d);
  return v == M3_F32 || v == M3_BF16;
}

// Shape checks shared by prefill and its workspace query.
m3_status check_prefill_shape(const m3_dims* d, int chunk, m3_dtype dtype) {
  if (!d) return M3_ERR_INVALID_VALUE;
  if (dtype != M3_F32 && dtype != M3_BF16) return M3_ERR_INVALID_VALUE;
  if (d->batch < 0 || d->seqlen < 0 || d->nheads < 1 || d->headdim_p < 1 || d->dstate_n < 2 ||
      d->rank_r < 1 || (d->dstate_n % 2) != 0)
    return M3_ERR_INVALID_VALUE;
  if (chunk < 1) return M3_ERR_INVALID_VALUE;
  if (!valid_p(d->headdim_p) || !valid_r(d->rank_r)) return M3_ERR_NOT_SUPPORTED;
  const int nmul = dtype == M3_BF16 ? 32 : 16;
  if (d->dstate_n < 16 || d->dstate_n > 256 || d->dstate_n % nmul != 0) return M3_ERR_NOT_SUPPORTED;
  if (chunk % 16 != 0 || chunk > m3::kLMax || chunk * d->rank_r > m3::kLRMax)
    return M3_ERR_NOT_SUPPORTED;
  const int64_t nC = (d->seqlen + chunk - 1) / chunk;
  if (d->seqlen > INT_MAX || d->batch > INT_MAX || d->nheads > INT_MAX ||
      d->batch * d->nheads * (nC > 0 ? nC : 1) > INT_MAX)
    return M3_ERR_NOT_SUPPORTED;
  const int es = (int)esize_of(dtype);
  const m3::PrefillLayout lay = m3::prefill_layout(chunk, (int)d->rank_r, (int)d->dstate_n,
                                                   (int)d->headdim_p, es);
  if (lay.total > m3::kLdsLimit) return M3_ERR_NOT_SUPPORTED;
  if (!m3::prefill_shape_fits(chunk, (int)d->rank_r, (int)d->dstate_n, (int)d->headdim_p,
                              (int)d->nheads, es))
    return M3_ERR_NOT_SUPPORTED;
  return M3_SUCCESS;
}

struct WsCarve {
  size_t grid, off_slots, off_cont, total;
};

// The counters come first, at offsets that do not depend on the shape (see
// kStatusWord): the ticket counters, the error word and the
// finished-workgroup count, then from word kStatusWord one status word per
// workgroup (segment).  The segments' slots (aggregate, exit state, rotation
// and decay) start at kSlotsMinBytes or past the counters, whichever is
// later, then the continuation entry states.  A call has at most 256 + units
// workgroups when units < 256 and exactly units otherwise, so calls with at
// most 1792 units keep their counters below 8 KiB and never store states
// where any call keeps counters.
WsCarve carve(const m3_dims* d, int chunk, m3_dtype /*dtype*/) {
  WsCarve w;
  const size_t units = (size_t)d->batch * d->nheads;
  const int nC = (int)((d->seqlen + chunk - 1) / chunk);
  const int K = m3::prefill_segment_chunks((int)d->batch, (int)d->nheads, nC > 0 ? nC : 1);
  w.grid = units * (size_t)((nC + K - 1) / K);
  const size_t counters = round256((m3::kStatusWord + w.grid) * sizeof(int));
  w.off_slots = counters > m3::kSlotsMinBytes ? counters : m3::kSlotsMinBytes;
  const size_t np = (size_t)d->dstate_n * d->headdim_p;
  w.off_cont = w.off_slots + round256(w.grid * m3::prefill_slot_floats((int)d->dstate_n,
                                                                       (int)d->headdim_p) *
                                      sizeof(float));
  w.total = round256(w.off_cont + units * np * sizeof(float));
  return w;
}

}  // namespace

extern "C" {

int m3_version(void) { return M3SSM_VERSION; }

const char* m3_status_string(m3_status s) {
  switch (enum_bits(&s)) {
    case M3_SUCCESS: return "M3_SUCCESS: no error";
    case M3_ERR_INVALID_VALUE:
      return "M3_ERR_INVALID_VALUE: null pointer, bad size, misaligned pointer or bad chunk";
    case M3_ERR_NOT_SUPPORTED: return "M3_ERR_NOT_SUPPORTED: shape outside the compiled set";
    case M3_ERR_WORKSPACE: return "M3_ERR_WORKSPACE: workspace missing or too small";
    case M3_ERR_HIP: return "M3_ERR_HIP: a HIP runtime call or kernel launch failed";
    case M3_ERR_CHAIN:
      return "M3_ERR_CHAIN: a prefill chain wait timed out (outputs NaN) or the workspace "
             "counters were dirty on entry";
  }
  return "unknown m3_status";
}

m3_status m3_prefill_workspace_error(void* workspace, size_t workspace_bytes, int clear,
                                     int* error_word, void* stream) {
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < 16) return M3_ERR_INVALID_VALUE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int* word = static_cast<int*>(workspace) + 1;  // word 1 of the counters
  int host = 0;
  if (hipMemcpyAsync(&host, word, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return M3_ERR_HIP;
  if (error_word) *error_word = host;
  if (host != 0 && clear) {
    static const int kZero = 0;
    if (hipMemcpyAsync(word, &kZero, sizeof(int), hipMemcpyHostToDevice, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return M3_ERR_HIP;
  }
  return host == 0 ? M3_SUCCESS : M3_ERR_CHAIN;
}

size_t m3_prefill_workspace_size(const m3_dims* dims, int chunk, m3_dtype dtype) {
  if (!dtype_ok(&dtype)) return 0;
  if (check_prefill_shape(dims, chunk, dtype) != M3_SUCCESS) return 0;
  if (dims->batch == 0 || dims->seqlen == 0) return 0;
  return carve(dims, chunk, dtype).total;
}

}  // extern "C"

namespace {

// ---- scratch of the no-allocation entry point -----------------------------
// A file-scope device array: each GPU the library runs on holds its own copy
// (kNoAllocScratchBytes) until the process ends.  Host code never uses the
// array's name as an address: the device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and kept here.
constexpr size_t kNoAllocScratchBytes = M3_PREFILL_NOALLOC_SCRATCH_BYTES;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, or nullptr on a HIP error.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

namespace m3 {

hipError_t lds_limit(const void* fn, size_t bytes) {
  struct Entry {
    const void* fn;
    int dev;
    size_t bytes;
  };
  static std::mutex mu;
  static Entry table[256];
  static int used = 0;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  int i = 0;
  while (i < used && !(table[i].fn == fn && table[i].dev == dev)) ++i;
  if (i < used && table[i].bytes >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  if (i == used) {
    if (used == 256) return hipSuccess;  // table full: correct, only not cached
    table[used++] = Entry{fn, dev, bytes};
  } else {
    table[i].bytes = bytes;
  }
  return hipSuccess;
}

}  // namespace m3

namespace {

// Zero n int32 words (the chain counters of the no-allocation entry point's
// scratch); a plain fill kernel, so a caller may capture the call into a graph.
__global__ void zero_words_kernel(int* w, int n) {
  for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < n; i += (int)(gridDim.x * blockDim.x))
    w[i] = 0;
}

m3_status prefill_impl(const m3_dims* dims, m3_dtype dtype, int chunk, const float* h0,
                       const void* x_prev, const void* B_prev, const void* x, const float* dt,
                       const float* A, const float* lam, const float* theta, const void* B,
                       const void* C, void* y, float* h_final, void* workspace,
                       size_t workspace_bytes, void* stream, bool noalloc = false) {
  const m3_status st = check_prefill_shape(dims, chunk, dtype);
  if (st != M3_SUCCESS) return st;
  const bool work = dims->batch > 0 && dims->seqlen > 0;
  const uintptr_t es = esize_of(dtype);
  if (work) {
    // lam and theta are optional (the exponential-Euler rule, a real state)
    if (!x || !dt || !A || !B || !C || !y) return M3_ERR_INVALID_VALUE;
    // x, B, C and theta are read in 16-byte vectors
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(theta, 16) ||
        !aligned(y, es) || !aligned(dt, 4) || !aligned(A, 4) || !aligned(lam, 4))
      return M3_ERR_INVALID_VALUE;
  }
  if (h_final && !aligned(h_final, 4)) return M3_ERR_INVALID_VALUE;
  // the continuation inputs: the previous token's x and B come together
  if ((x_prev == nullptr) != (B_prev == nullptr)) return M3_ERR_INVALID_VALUE;
  if ((h0 && !aligned(h0, 4)) || (x_prev && !aligned(x_prev, es)) ||
      (B_prev && !aligned(B_prev, es)))
    return M3_ERR_INVALID_VALUE;
  // h_final may be h0 itself but must not partially overlap it
  if (h0 && h_final && h0 != h_final) {
    const size_t hbytes =
        (size_t)dims->batch * dims->nheads * dims->dstate_n * dims->headdim_p * sizeof(float);
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(h0), a1 = reinterpret_cast<uintptr_t>(h_final);
    if (a0 < a1 + hbytes && a1 < a0 + hbytes) return M3_ERR_INVALID_VALUE;
  }
  size_t need = 0;
  WsCarve w = {};
  if (work) {
    w = carve(dims, chunk, dtype);
    need = w.total;
    if (noalloc) {
      // the library's scratch instead of a caller's workspace: the first HIP
      // call of a no-allocation call, after every argument check
      if (need > kNoAllocScratchBytes) return M3_ERR_WORKSPACE;
      workspace = device_scratch();
      if (!workspace) return M3_ERR_HIP;
      workspace_bytes = kNoAllocScratchBytes;
    }
    if (!workspace || workspace_bytes < need) return M3_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return M3_ERR_INVALID_VALUE;
  }
  if (dims->batch == 0) return M3_SUCCESS;

  m3::PrefillArgs a = {};
  a.nb = (int)dims->batch;
  a.T = (int)dims->seqlen;
  a.H = (int)dims->nheads;
  a.P = (int)dims->headdim_p;
  a.N = (int)dims->dstate_n;
  a.R = (int)dims->rank_r;
  a.L = chunk;
  a.nC = (int)((dims->seqlen + chunk - 1) / chunk);
  a.K = m3::prefill_segment_chunks(a.nb, a.H, a.nC > 0 ? a.nC : 1);
  a.nSeg = (a.nC + a.K - 1) / a.K;
  a.x = x;
  a.dt = dt;
  a.A = A;
  a.lam = lam;
  a.theta = theta;
  a.B = B;
  a.C = C;
  a.h0 = h0;
  a.x_prev = x_prev;
  a.B_prev = B_prev;
  a.cont = (h0 != nullptr || x_prev != nullptr) ? 1 : 0;
  a.y = y;
  a.h_final = h_final;
  if (work) {
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    a.slots = reinterpret_cast<float*>(ws + w.off_slots);
    a.cont_entry = reinterpret_cast<float*>(ws + w.off_cont);
    a.ticket = reinterpret_cast<int*>(ws);
    a.err = a.ticket + 1;
    a.done = a.ticket + 2;
    a.status = a.ticket + m3::kStatusWord;
    a.ncls = m3::prefill_ticket_classes((long long)a.nb * a.H);
  }
  if (noalloc && work) {
    const int nwords = (int)(m3::kStatusWord + w.grid);
    const int blocks = (nwords + 255) / 256;
    hipLaunchKernelGGL(zero_words_kernel, dim3(blocks < 1024 ? blocks : 1024), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a.ticket, nwords);
    if (hipGetLastError() != hipSuccess) return M3_ERR_HIP;
  }
  const hipError_t e = m3::launch_prefill(a, dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? M3_SUCCESS : M3_ERR_HIP;
}

}  // namespace

extern "C" {

m3_status m3_prefill(const m3_dims* dims, m3_dtype dtype, int chunk, const void* x,
                     const float* dt, const float* A, const float* lam, const float* theta,
                     const void* B, const void* C, void* y, float* h_final, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!dtype_ok(&dtype)) return M3_ERR_INVALID_VALUE;
  return prefill_impl(dims, dtype, chunk, nullptr, nullptr, nullptr, x, dt, A, lam, theta, B, C,
                      y, h_final, workspace, workspace_bytes, stream);
}

m3_status m3_prefill_noalloc(const m3_dims* dims, m3_dtype dtype, int chunk, const void* x,
                             const float* dt, const float* A, const float* lam,
                             const float* theta, const void* B, const void* C, void* y,
                             float* h_final, void* stream) {
  if (!dtype_ok(&dtype)) return M3_ERR_INVALID_VALUE;
  return prefill_impl(dims, dtype, chunk, nullptr, nullptr, nullptr, x, dt, A, lam, theta, B, C,
                      y, h_final, nullptr, 0, stream, true);
}

m3_status m3_prefill_from_state(const m3_dims* dims, m3_dtype dtype, int chunk, const float* h0,
                                const void* x_prev, const void* B_prev, const void* x,
                                const float* dt, const float* A, const float* lam,
                                const float* theta, const void* B, const void* C, void* y,
                                float* h_final, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (!dtype_ok(&dtype)) return M3_ERR_INVALID_VALUE;
  return prefill_impl(dims, dtype, chunk, h0, x_prev, B_prev, x, dt, A, lam, theta, B, C, y,
                      h_final, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// m3_decode_step and m3_decode_step_mfma: the same checks, then the vector
// kernel or the matrix-core one.
m3_status decode_impl(const m3_dims* dims, m3_dtype dtype, const float* h_in, float* h_out,
                      const void* x_t, const void* x_prev, const void* B_t, const void* B_prev,
                      const void* C_t, const float* dt, const float* A, const float* lam,
                      const float* theta, void* y_t, void* stream, bool mfma) {
  if (!dtype_ok(&dtype)) return M3_ERR_INVALID_VALUE;
  if (!dims) return M3_ERR_INVALID_VALUE;
  if (dtype != M3_F32 && dtype != M3_BF16) return M3_ERR_INVALID_VALUE;
  const m3_dims* d = dims;
  if (d->batch < 0 || d->nheads < 1 || d->headdim_p < 1 || d->dstate_n < 2 || d->rank_r < 1 ||
      (d->dstate_n % 2) != 0)
    return M3_ERR_INVALID_VALUE;
  if (!valid_p(d->headdim_p) || !valid_r(d->rank_r)) return M3_ERR_NOT_SUPPORTED;
  if (d->dstate_n > 256 || d->dstate_n > m3::decode_max_n((int)d->headdim_p))
    return M3_ERR_NOT_SUPPORTED;
  if (mfma && !m3::decode_mfma_shape((int)d->rank_r, (int)d->dstate_n, (int)d->headdim_p))
    return M3_ERR_NOT_SUPPORTED;
  if (d->batch * d->nheads > INT_MAX) return M3_ERR_NOT_SUPPORTED;
  if (d->batch == 0) return M3_SUCCESS;
  // lam and theta are optional; without lam x_prev and B_prev are not read
  const void* ptrs[] = {h_in, h_out, x_t, B_t, C_t, dt, A, y_t};
  for (const void* p : ptrs)
    if (!p) return M3_ERR_INVALID_VALUE;
  if (lam && (!x_prev || !B_prev)) return M3_ERR_INVALID_VALUE;
  // state rows in float4, x in 4-element vectors, B and C in rotation pairs
  const uintptr_t es = esize_of(dtype);
  if (!aligned(h_in, 16) || !aligned(h_out, 16) || !aligned(x_t, 4 * es) ||
      !aligned(x_prev, 4 * es) || !aligned(B_t, 2 * es) || !aligned(B_prev, 2 * es) ||
      !aligned(C_t, 2 * es) || !aligned(y_t, es) || !aligned(dt, 4) || !aligned(A, 4) ||
      !aligned(lam, 4) || !aligned(theta, 4))
    return M3_ERR_INVALID_VALUE;
  // h_out may equal h_in but must not partially overlap it
  const size_t hbytes = (size_t)d->batch * d->nheads * d->dstate_n * d->headdim_p * sizeof(float);
  const uintptr_t hi = reinterpret_cast<uintptr_t>(h_in), ho = reinterpret_cast<uintptr_t>(h_out);
  if (hi != ho && hi < ho + hbytes && ho < hi + hbytes) return M3_ERR_INVALID_VALUE;

  m3::DecodeArgs a = {};
  a.S = (int)d->batch;
  a.H = (int)d->nheads;
  a.P = (int)d->headdim_p;
  a.N = (int)d->dstate_n;
  a.R = (int)d->rank_r;
  a.h_in = h_in;
  a.h_out = h_out;
  a.x_t = x_t;
  a.x_prev = x_prev;
  a.B_t = B_t;
  a.B_prev = B_prev;
  a.C_t = C_t;
  a.dt = dt;
  a.A = A;
  a.lam = lam;
  a.theta = theta;
  a.y = y_t;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = mfma ? m3::launch_decode_mfma(a, dtype, st) : m3::launch_decode(a, dtype, st);
  return e == hipSuccess ? M3_SUCCESS : M3_ERR_HIP;
}

}  // namespace

extern "C" {

m3_status m3_decode_step(const m3_dims* dims, m3_dtype dtype, const float* h_in, float* h_out,
                         const void* x_t, const void* x_prev, const void* B_t,
                         const void* B_prev, const void* C_t, const float* dt, const float* A,
                         const float* lam, const float* theta, void* y_t, void* stream) {
  return decode_impl(dims, dtype, h_in, h_out, x_t, x_prev, B_t, B_prev, C_t, dt, A, lam, theta,
                     y_t, stream, false);
}

m3_status m3_decode_step_mfma(const m3_dims* dims, m3_dtype dtype, const float* h_in,
                              float* h_out, const void* x_t, const void* x_prev, const void* B_t,
                              const void* B_prev, const void* C_t, const float* dt,
                              const float* A, const float* lam, const float* theta, void* y_t,
                              void* stream) {
  return decode_impl(dims, dtype, h_in, h_out, x_t, x_prev, B_t, B_prev, C_t, dt, A, lam, theta,
                     y_t, stream, true);
}

}  // extern "C"

// ---- block-side passes ------------------------------------------------------

namespace {

m3_status check_block_dims(const m3_dims* d, m3_dtype dtype) {
  if (!d) return M3_ERR_INVALID_VALUE;
  if (dtype != M3_F32 && dtype != M3_BF16) return M3_ERR_INVALID_VALUE;
  if (d->batch < 0 || d->seqlen < 0 || d->nheads < 1 || d->headdim_p < 1 || d->dstate_n < 1 ||
      d->rank_r < 1)
    return M3_ERR_INVALID_VALUE;
  if (!valid_p(d->headdim_p) || !valid_r(d->rank_r)) return M3_ERR_NOT_SUPPORTED;
  // a B / C row must be a power-of-two number of 16-byte vectors
  const int64_t n = d->dstate_n;
  if (n != 16 && n != 32 && n != 64 && n != 128 && n != 256) return M3_ERR_NOT_SUPPORTED;
  if (d->batch > INT32_MAX || d->seqlen > INT32_MAX || d->nheads > INT32_MAX ||
      (double)d->batch * (double)d->seqlen * (double)d->nheads * (double)d->rank_r * 256.0 >
          9.0e15)
    return M3_ERR_NOT_SUPPORTED;
  return M3_SUCCESS;
}

m3::BlockArgs block_args(const m3_dims* d) {
  m3::BlockArgs a = {};
  a.rows = (size_t)d->batch * (size_t)d->seqlen * (size_t)d->nheads;
  a.H = (int)d->nheads;
  a.P = (int)d->headdim_p;
  a.N = (int)d->dstate_n;
  a.R = (int)d->rank_r;
  return a;
}

}  // namespace

extern "C" {

m3_status m3_block_prepass(const m3_dims* dims, m3_dtype dtype, const void* x, const void* B,
                           const void* C, const float* norm_B, const float* norm_C,
                           const float* bias_B, const float* bias_C, const float* up, float eps,
                           void* x_out, void* B_out, void* C_out, void* stream) {
  if (!dtype_ok(&dtype)) return M3_ERR_INVALID_VALUE;
  const m3_status st = check_block_dims(dims, dtype);
  if (st != M3_SUCCESS) return st;
  if (!(eps >= 0.f) || !(eps < 3.0e38f)) return M3_ERR_INVALID_VALUE;  // also rejects NaN
  m3::BlockArgs a = block_args(dims);
  if (a.rows == 0) return M3_SUCCESS;
  const void* vec[] = {x, B, C, x_out, B_out, C_out};
  for (const void* p : vec)
    if (!p || !aligned(p, 16)) return M3_ERR_INVALID_VALUE;
  // weights are read in 16-byte vectors too
  const float* wts[] = {norm_B, norm_C, bias_B, bias_C, up};
  for (const float* p : wts)
    if (!p || !aligned(p, 16)) return M3_ERR_INVALID_VALUE;
  a.eps = eps;
  a.x = x;
  a.B = B;
  a.C = C;
  a.norm_B = norm_B;
  a.norm_C = norm_C;
  a.bias_B = bias_B;
  a.bias_C = bias_C;
  a.up = up;
  a.x_out = x_out;
  a.B_out = B_out;
  a.C_out = C_out;
  const hipError_t e = m3::launch_block_prepass(a, dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? M3_SUCCESS : M3_ERR_HIP;
}

m3_status m3_block_postpass(const m3_dims* dims, m3_dtype dtype, const void* y,
                            const float* down, void* y_out, void* stream) {
  if (!dtype_ok(&dtype)) return M3_ERR_INVALID_VALUE;
  const m3_status st = check_block_dims(dims, dtype);
  if (st != M3_SUCCESS) return st;
  m3::BlockArgs a = block_args(dims);
  if (a.rows == 0) return M3_SUCCESS;
  if (!y || !y_out || !aligned(y, 16) || !aligned(y_out, 16)) return M3_ERR_INVALID_VALUE;
  if (!down || !aligned(down, 16)) return M3_ERR_INVALID_VALUE;
  a.y = y;
  a.down = down;
  a.y_out = y_out;
  const hipError_t e = m3::launch_block_postpass(a, dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? M3_SUCCESS : M3_ERR_HIP;
}

}  // extern "C"

// ---- gradients ----------------------------------------------------------------

namespace {

m3_status check_backward_dims(const m3_dims* d, m3_dtype dtype) {
  if (!d) return M3_ERR_INVALID_VALUE;
  if (dtype != M3_F32 && dtype != M3_BF16) return M3_ERR_INVALID_VALUE;
  if (d->batch < 0 || d->seqlen < 0 || d->nheads < 1 || d->headdim_p < 1 || d->dstate_n < 2 ||
      d->rank_r < 1 || (d->dstate_n % 2) != 0)
    return M3_ERR_INVALID_VALUE;
  if (!valid_p(d->headdim_p) || !valid_r(d->rank_r)) return M3_ERR_NOT_SUPPORTED;
  // a power-of-two state size with N * P <= 8192: one workgroup of
  // (N/2) (P/8) <= 512 threads per token-head
  const int64_t n = d->dstate_n;
  if ((n != 16 && n != 32 && n != 64 && n != 128 && n != 256) || n * d->headdim_p > 8192)
    return M3_ERR_NOT_SUPPORTED;
  if (d->batch > INT32_MAX || d->seqlen > INT32_MAX || d->nheads > INT32_MAX ||
      (double)d->batch * (double)d->seqlen * (double)d->nheads > 2.0e9)
    return M3_ERR_NOT_SUPPORTED;
  // the time loops address one sequence's tokens with 32-bit buffer offsets
  const double es = dtype == M3_BF16 ? 2.0 : 4.0;
  const double row = (double)d->nheads * d->rank_r * (d->dstate_n > d->headdim_p ? d->dstate_n
                                                                                 : d->headdim_p);
  if ((double)d->seqlen * row * es >= 2147483648.0 ||
      (double)d->seqlen * d->nheads * (d->dstate_n / 2) * 4.0 >= 2147483648.0 ||
      (double)d->seqlen * d->dstate_n * d->headdim_p * 4.0 >= 2147483648.0)
    return M3_ERR_NOT_SUPPORTED;
  return M3_SUCCESS;
}

struct BwCarve {
  int S;  // segment length of the checkpointed path, 0 for per-token states
  int L;  // chunk length of the chunked path, 0 for the other two
  size_t off_gs, off_dAc, off_dseg, off_psi, total;
};

// The states: with chunks of L tokens (N = P = 64) the entry state of every
// chunk and the next, the exit adjoint of every chunk, per chunk its
// rotation and decay and per token four partial scalars; else with segments
// of S tokens one entry state and one exit adjoint per segment; else h_t and
// G_t of every token.
BwCarve bw_carve(const m3_dims* d, m3_dtype dtype) {
  BwCarve w;
  w.L = 0;
  if (m3::bw_chunked_shape((int)d->rank_r, (int)d->dstate_n, (int)d->headdim_p)) {
    w.S = 0;
    w.L = 64 / (int)d->rank_r;
    const size_t units = (size_t)d->batch * d->nheads;
    const size_t nC = (size_t)(d->seqlen + w.L - 1) / w.L;
    const size_t np = (size_t)d->dstate_n * d->headdim_p;
    w.off_gs = round256(units * (nC + 1) * np * sizeof(float));
    w.off_dAc = w.off_gs + round256(units * nC * np * sizeof(float));
    w.off_dseg = w.off_dAc + round256(4 * units * d->seqlen * sizeof(float));
    w.off_psi = w.off_dseg + round256(units * nC * 65 * sizeof(float));
    w.total = w.off_psi;
    return w;
  }
  w.S = m3::bw_segment_len((int)d->rank_r, (int)d->dstate_n, (int)d->headdim_p,
                           (int)esize_of(dtype));
  const size_t slots = w.S ? (size_t)(d->seqlen + w.S - 1) / w.S : (size_t)d->seqlen;
  const size_t states = (size_t)d->batch * d->nheads * slots * d->dstate_n * d->headdim_p;
  w.off_gs = round256(states * sizeof(float));
  w.off_dAc = w.off_gs + round256(states * sizeof(float));
  w.off_dseg = w.off_dAc + round256((size_t)d->batch * d->seqlen * d->nheads * sizeof(float));
  // per segment: decay and one rotation angle per row pair
  const size_t segs = w.S ? (size_t)d->batch * d->nheads * slots : 0;
  w.off_psi = w.off_dseg + round256(segs * sizeof(float));
  w.total = w.off_psi + round256(segs * (d->dstate_n / 2) * sizeof(float));
  return w;
}

}  // namespace

extern "C" {

size_t m3_backward_workspace_size(const m3_dims* dims, m3_dtype dtype) {
  if (!dtype_ok(&dtype)) return 0;
  if (check_backward_dims(dims, dtype) != M3_SUCCESS) return 0;
  if (dims->batch == 0 || dims->seqlen == 0) return 0;
  return bw_carve(dims, dtype).total;
}

m3_status m3_backward(const m3_dims* dims, m3_dtype dtype, const void* x, const float* dt,
                      const float* A, const float* lam, const float* theta, const void* B,
                      const void* C, const void* dy, const float* dh_final, float* dx,
                      float* ddt, float* dA, float* dlam, float* dtheta, float* dB, float* dC,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(&dtype)) return M3_ERR_INVALID_VALUE;
  const m3_status st = check_backward_dims(dims, dtype);
  if (st != M3_SUCCESS) return st;
  const uintptr_t es = esize_of(dtype);
  if (!dA || !aligned(dA, 4)) return M3_ERR_INVALID_VALUE;
  // with no tokens only dA is written (the other arrays may be empty)
  if (dims->batch > 0 && dims->seqlen > 0) {
    // x and dy are read in 16-byte vectors
    if (!x || !dy || !aligned(x, 16) || !aligned(dy, 16)) return M3_ERR_INVALID_VALUE;
    const void* in_t[] = {B, C};
    const void* f32[] = {dt, A, lam, theta, dx, ddt, dlam, dtheta, dB, dC};
    for (const void* p : in_t)
      if (!p || !aligned(p, es)) return M3_ERR_INVALID_VALUE;
    for (const void* p : f32)
      if (!p || !aligned(p, 4)) return M3_ERR_INVALID_VALUE;
    if (dh_final && !aligned(dh_final, 4)) return M3_ERR_INVALID_VALUE;
  }
  m3::BackwardArgs a = {};
  a.nb = (int)dims->batch;
  a.T = (int)dims->seqlen;
  a.H = (int)dims->nheads;
  a.P = (int)dims->headdim_p;
  a.N = (int)dims->dstate_n;
  a.R = (int)dims->rank_r;
  a.dA = dA;
  if (a.nb == 0 || a.T == 0) {
    // no tokens: the per-token gradients are empty and dA sums nothing
    const hipError_t e = m3::launch_backward(a, dtype, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? M3_SUCCESS : M3_ERR_HIP;
  }
  const BwCarve w = bw_carve(dims, dtype);
  if (!workspace || workspace_bytes < w.total) return M3_ERR_WORKSPACE;
  a.S = w.S;
  a.L = w.L;
  if (!aligned(workspace, 256)) return M3_ERR_INVALID_VALUE;
  a.x = x;
  a.B = B;
  a.C = C;
  a.dy = dy;
  a.dt = dt;
  a.A = A;
  a.lam = lam;
  a.theta = theta;
  a.dh_final = dh_final;
  a.dx = dx;
  a.ddt = ddt;
  a.dA = dA;
  a.dlam = dlam;
  a.dtheta = dtheta;
  a.dB = dB;
  a.dC = dC;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  a.hs = reinterpret_cast<float*>(ws);
  a.gs = reinterpret_cast<float*>(ws + w.off_gs);
  a.dAc = reinterpret_cast<float*>(ws + w.off_dAc);
  a.dseg = reinterpret_cast<float*>(ws + w.off_dseg);
  a.psi = reinterpret_cast<float*>(ws + w.off_psi);
  const hipError_t e = m3::launch_backward(a, dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? M3_SUCCESS : M3_ERR_HIP;
}

}  // extern "C"
