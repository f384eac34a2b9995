/*
 * m3ssm.h -- C ABI of libm3ssm: the Mamba-3 SSM layer recurrence on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (per batch b and head h, t = 0..T-1):
 *
 *   h_t = alpha_t R_t ( h_{t-1} + (1 - lam_t) dt_t B_{t-1} x_{t-1}^T )
 *         + lam_t dt_t B_t x_t^T
 *   y_t = C_t^T h_t
 *
 * with alpha_t = exp(dt_t * A) and R_t the block-diagonal rotation whose 2x2
 * block for rows (2k, 2k+1) is [[cos p, -sin p], [sin p, cos p]], p = dt_t *
 * theta_t[k].  This is the exponential-trapezoidal rule (Mamba-3 paper
 * summary, aipaper.cc, "Mathematical formulas", Proposition 1: alpha =
 * e^{dt A}, beta = (1-lam) dt alpha, gamma = lam dt; Mamba-3 explainer,
 * yunpan.plus, "first improvement") applied to the complex transition
 * A + i theta, realised as 2x2 rotations (explainer, "second improvement";
 * paper summary, Proposition 3: the rotations can be moved onto B and C as a
 * data-dependent RoPE).  MIMO (paper summary, item 3; explainer, "third
 * improvement"): x_t is P x R and B_t, C_t are N x R, so B x^T is a rank-R
 * product and y_t is R x P.  h_{-1} = 0 and B_{-1} x_{-1}^T = 0.
 *
 * Reduced forms.  Every entry point takes lam and theta as optional: a NULL
 * lam means lam = 1, the exponential-Euler rule -- the previous-input term
 * vanishes and the update is Mamba-2's h = e^{dt A} h + dt B x^T (paper
 * summary, Proposition 1 with lam = 1; paper translation, Remark 5) -- and a
 * NULL theta means theta = 0, a real-valued state with no rotation (the
 * complex transition of the explainer's "second improvement" switched off).
 * Both NULL is the Mamba-2 recurrence on the same kernels.
 *
 * Layouts (row-major, dense, no strides).  T is the storage type chosen by
 * m3_dtype (float or bfloat16) for x, B, C and y; everything else is float:
 *   x, y       [batch, T, H, R, P]   (x_t stored as its transpose, P contiguous)
 *   B, C       [batch, T, H, R, N]   (N contiguous)
 *   dt, lam    [batch, T, H]         (dt > 0 already softplus'd; lam in [0,1])
 *   theta      [batch, T, H, N/2]    (angle rate per rotation pair)
 *   A          [H]                   (A <= 0, constant in time)
 *   h_final    [batch, H, N, P]      (state after the last token, float)
 *
 * Ownership and threading: every pointer is caller-owned DEVICE memory on the
 * current HIP device, aligned to its element size and further as each call
 * states (vector loads).  The library allocates nothing and, apart from the
 * per-GPU scratch of m3_prefill_noalloc, keeps no mutable global state;
 * calls enqueue work on `stream` (a hipStream_t; NULL = the default stream)
 * and return without synchronising.  Calls on different streams that write
 * different buffers may overlap.
 *
 * Errors: every argument is validated on the host before anything is
 * enqueued; an invalid call returns an error code and enqueues nothing.  A
 * failed kernel launch returns M3_ERR_HIP.  Faults inside kernels surface, as
 * with any HIP kernel, at the caller's next synchronisation.  Data
 * preconditions (A <= 0, dt > 0, lam in [0,1], finite inputs) are documented,
 * not checked.  No C++ exception crosses this interface.
 */
#ifndef M3SSM_H_
#define M3SSM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define M3SSM_VERSION 150 /* 1.5.0 */

typedef enum {
  M3_SUCCESS = 0,
  M3_ERR_INVALID_VALUE = 1, /* null pointer, bad size, misalignment, bad chunk */
  M3_ERR_NOT_SUPPORTED = 2, /* valid but outside the compiled shape set */
  M3_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
  M3_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed */
  M3_ERR_CHAIN = 5          /* a prefill workspace's error word is set (see
                               m3_prefill_workspace_error) */
} m3_status;

typedef enum {
  M3_F32 = 0, /* x, B, C, y stored as float */
  M3_BF16 = 1 /* x, B, C, y stored as bfloat16; accumulation stays float */
} m3_dtype;

typedef struct {
  int64_t batch;     /* sequences (>= 0) */
  int64_t seqlen;    /* T, tokens per sequence (>= 0; ignored by decode) */
  int64_t nheads;    /* H (>= 1) */
  int64_t headdim_p; /* P: 16, 32, 64 or 128 */
  int64_t dstate_n;  /* N: even; 16..256 and a multiple of 16 (bf16 prefill: of 32) */
  int64_t rank_r;    /* R: 1, 2 or 4 (MIMO rank) */
} m3_dims;

/* Library version (M3SSM_VERSION of the compiled library). */
int m3_version(void);

/* Static, NUL-terminated description of a status code. */
const char* m3_status_string(m3_status status);

/*
 * Bytes of device workspace m3_prefill needs for these dims, chunk and dtype;
 * 0 if the combination is invalid or unsupported (m3_prefill then says why).
 * Host only; enqueues nothing.
 */
size_t m3_prefill_workspace_size(const m3_dims* dims, int chunk, m3_dtype dtype);

/*
 * Chunked prefill of the whole sequence: writes y for every token and, if
 * h_final is not NULL, the state after the last token.
 *
 * chunk: tokens per chunk, a multiple of 16 with 16 <= chunk <= 128 and
 * chunk * R <= 256.  The result does not depend on the chunk beyond float
 * rounding: inside a chunk the recurrence is evaluated in its parallel
 * (structured-mask) form -- the decay matrix times the 2-band trapezoid
 * matrix (Mamba-3 paper translation, sz-guanghua.com.cn, section 3.1,
 * equation 7) with B and C rotated by the cumulative angles (data-dependent
 * RoPE, paper summary Proposition 3) -- and chunks are chained by the
 * recurrence on the state (explainer: parallel inside a chunk, recurrent
 * across chunks).  T need not be a multiple of chunk.
 *
 * Alignment: x, B, C and theta 16 bytes; y, dt, lam, A and h_final one
 * element.
 *
 * workspace: device scratch of at least m3_prefill_workspace_size() bytes,
 * 256-byte aligned, owned by the caller.  A call runs one workgroup per
 * segment: with units = batch * nheads and nC = ceil(seqlen / chunk), a
 * segment is K = min(nC, max(1, ceil(nC * units / 256))) chunks and there are
 * G = units * ceil(nC / K) of them (G < 256 + units, and G = units when
 * units >= 256).  The workspace starts with the chain's int32 counters:
 * the work-ticket counters of up to 8 classes of workgroups (class c's at
 * word 32 c, so word 0 is class 0's), word 1 the error word, word 2 the
 * finished-workgroup count, the other words below 256 unused, then from
 * word 256 one status word per segment: 1024 + 4 G bytes.  From byte 8192
 * or from the first 256-byte boundary past the counters (whichever is
 * later) it holds one slot per segment (the map from its entry to its exit
 * state, then its exit state) and the entry state of each sequence.  A call
 * needs its counters zero on entry and leaves them zero (its last workgroup
 * resets them), so a buffer zero-filled once serves every later call as
 * long as batch * nheads <= 1792 (then 256 + G <= 2048 words), or as long
 * as no call has more segments than the call before it on this buffer;
 * otherwise zero the counter bytes before the call.
 *
 * Chain errors.  The error word is left nonzero, and stays so until cleared
 * (m3_prefill_workspace_error), when:
 *  1  a segment waited beyond its bounded spin (about a quarter of a second)
 *     for a predecessor.  Its entry state is then unknown: it continues from
 *     NaN, so its y, every state it hands on (hence the rest of that
 *     sequence's y) and h_final are NaN.  (Two shapes also have a bounded
 *     wait between the waves of one workgroup, for scores one wave hands to
 *     another: bfloat16, R = 1, chunk 64 with N = P = 64 (the single-pass
 *     kernel) or with N = 128, P <= 64.  It sets this word if it runs out,
 *     which it cannot while the workgroup runs.)
 *  2  the counters were not zero on entry, as seen by a workgroup whose
 *     ticket lies past the grid (its class's ticket word was not zero) or
 *     whose own status word was not zero.  That workgroup computes nothing;
 *     others may then time out (1).  A nonzero finished-workgroup word (word 2) is not
 *     detected: it makes the reset at the end of the call happen early or
 *     not at all, so zero-fill the counter bytes after any call that did not
 *     finish normally.
 * m3_prefill returns once the work is enqueued, so it cannot report these;
 * m3_prefill_workspace_error reads the word back.  Concurrent calls need
 * distinct workspaces.
 *
 * Returns M3_SUCCESS once the kernel is enqueued (one launch per call).  y and h_final must not
 * overlap the inputs.  batch == 0 or seqlen == 0 enqueues nothing (h_final,
 * if given, is then zero-filled when seqlen == 0 and batch > 0).
 */
m3_status m3_prefill(const m3_dims* dims, m3_dtype dtype, int chunk, const void* x,
                     const float* dt, const float* A, const float* lam, const float* theta,
                     const void* B, const void* C, void* y, float* h_final, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Error word of a prefill workspace (see "Chain errors" above), read once
 * all work enqueued on `stream` so far has finished: this call synchronises
 * `stream` (so it cannot be captured into a graph).  Stores the word in
 * *error_word if error_word is not NULL and, if `clear` is nonzero and the
 * word is not 0, resets it to 0.  Returns M3_SUCCESS for a zero word,
 * M3_ERR_CHAIN for a nonzero one, M3_ERR_INVALID_VALUE if workspace is NULL,
 * not 256-byte aligned or smaller than 16 bytes (nothing is enqueued then),
 * and M3_ERR_HIP if a HIP call fails.
 */
m3_status m3_prefill_workspace_error(void* workspace, size_t workspace_bytes, int clear,
                                     int* error_word, void* stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): m3_prefill without a
 * workspace argument.  The same computation and kernels as m3_prefill; the
 * workspace is instead a scratch array inside the library, one per GPU (each
 * GPU the call runs on holds M3_PREFILL_NOALLOC_SCRATCH_BYTES of device
 * memory from its first such call until the process ends).  The call
 * allocates nothing: before the prefill kernel it clears the scratch's chain
 * counters with a small fill kernel (two launches per call; no memset), so
 * no state carries over between calls.  Every call on one GPU shares that
 * GPU's scratch: calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.  Returns
 * M3_ERR_WORKSPACE when the shape needs more workspace than the scratch holds
 * (m3_prefill_workspace_size(dims, chunk, dtype) >
 * M3_PREFILL_NOALLOC_SCRATCH_BYTES), before any HIP call; otherwise
 * arguments, layouts, alignment and errors are as for m3_prefill.  A chain
 * wait that times out shows as NaN outputs (the error word is cleared by the
 * next call and cannot be read back).
 */
#define M3_PREFILL_NOALLOC_SCRATCH_BYTES (32u << 20) /* 32 MiB per GPU */

m3_status m3_prefill_noalloc(const m3_dims* dims, m3_dtype dtype, int chunk, const void* x,
                             const float* dt, const float* A, const float* lam,
                             const float* theta, const void* B, const void* C, void* y,
                             float* h_final, void* stream);

/*
 * Prefill that continues a sequence: the same computation as m3_prefill, but
 * the recurrence starts from a given state and previous token instead of
 * zero, so a long prompt can be processed in pieces (or resumed from a cached
 * prefix) with the result of one call over the whole sequence, up to rounding.
 * The first token's update is then
 *
 *   h_0 = alpha_0 R_0 (h0 + (1-lam_0) dt_0 B_prev x_prev^T) + lam_0 dt_0 B_0 x_0^T
 *
 * -- the trapezoid rule's previous-input term (Mamba-3 paper summary,
 * Proposition 1; explainer, first improvement) with the previous token's
 * input, and the state and that term rotated together (explainer, second
 * improvement).  After a call over tokens 0..T1-1 the next piece passes
 * h0 = that call's h_final, x_prev = x[:, T1-1] and B_prev = B[:, T1-1]
 * (raw, unrotated), exactly as m3_decode_step does for one token.  The
 * chunked form chains chunks by the same recurrence on the state (explainer:
 * parallel inside a chunk, recurrent across chunks), so a piece boundary is
 * one more chunk boundary.
 *
 * h0:      [batch, nheads, N, P] fp32, unrotated frame, or NULL (zero state).
 * x_prev:  [batch, nheads, R, P] in x's dtype, or NULL (no previous token).
 * B_prev:  [batch, nheads, R, N] in x's dtype; NULL exactly when x_prev is.
 *
 * h_final may be h0 itself (the state is then updated in place) but must
 * not partially overlap it.  With seqlen == 0, h_final (if given) receives
 * h0, or zeros when h0 is NULL.  Everything else -- layouts, alignment,
 * workspace, errors -- is as for m3_prefill; the extra pointers need element
 * alignment.  With h0 or x_prev given the call enqueues two kernels: one
 * that writes each sequence's entry state into the workspace, then the
 * prefill kernel.  M3_ERR_INVALID_VALUE if exactly one of x_prev and B_prev
 * is NULL or h_final partially overlaps h0.
 */
m3_status m3_prefill_from_state(const m3_dims* dims, m3_dtype dtype, int chunk, const float* h0,
                                const void* x_prev, const void* B_prev, const void* x,
                                const float* dt, const float* A, const float* lam,
                                const float* theta, const void* B, const void* C, void* y,
                                float* h_final, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * One decode step for `batch` independent sequences (dims->seqlen ignored):
 *
 *   h_out = alpha R (h_in + (1-lam) dt B_prev x_prev^T) + lam dt B_t x_t^T
 *   y_t   = C_t^T h_out
 *
 * (the same recurrence, one token; the previous token's x and B are what the
 * trapezoid's beta term needs -- explainer, "first improvement"; the rank-R
 * product is the MIMO update -- paper summary, item 3).
 *
 * Layouts: h_in, h_out [batch, H, N, P] float, in the unrotated frame, and
 * h_out may equal h_in (in-place update); x_t, x_prev, y_t [batch, H, R, P];
 * B_t, B_prev, C_t [batch, H, R, N] (storage type from dtype); dt, lam
 * [batch, H]; theta [batch, H, N/2]; A [H].
 *
 * Alignment: h_in, h_out 16 bytes; x_t, x_prev four elements; B_t, B_prev,
 * C_t two elements; y_t, dt, lam, theta, A one element.
 *
 * First step of a fresh sequence: h_in = 0 and x_prev = B_prev = 0.  After a
 * prefill of T tokens: h_in = that call's h_final, x_prev = x_{T-1},
 * B_prev = B_{T-1} (the raw, unrotated inputs of the last prefilled token).
 *
 * lam and theta may be NULL (the reduced forms above).  Without lam the
 * previous token's term vanishes: x_prev and B_prev are not read and may be
 * NULL; with lam they are required.  Without theta, theta is not read.
 */
m3_status m3_decode_step(const m3_dims* dims, m3_dtype dtype, const float* h_in, float* h_out,
                         const void* x_t, const void* x_prev, const void* B_t,
                         const void* B_prev, const void* C_t, const float* dt, const float* A,
                         const float* lam, const float* theta, void* y_t, void* stream);

/*
 * The same decode step with the MIMO update's rank-2R product on the matrix
 * cores (the MIMO item of the paper summary, item 3, and the explainer's
 * "third improvement", which place that product on the tensor units): per
 * 16 x 16 tile of the state, v_mfma_f32_16x16x4_f32 accumulates
 * [x_prev | x_t] x [U | V]^T onto the rotated, decayed state.  Arguments,
 * layouts, alignment, reduced forms and errors are those of m3_decode_step;
 * results agree with it up to float rounding.  Shapes: R = 2 or 4, P = 64,
 * N a multiple of 16 up to 128; others return M3_ERR_NOT_SUPPORTED.  The
 * step is bound by the state's HBM traffic either way, so m3_decode_step
 * (vector ALU) stays the default.
 */
m3_status m3_decode_step_mfma(const m3_dims* dims, m3_dtype dtype, const float* h_in,
                              float* h_out, const void* x_t, const void* x_prev, const void* B_t,
                              const void* B_prev, const void* C_t, const float* dt,
                              const float* A, const float* lam, const float* theta, void* y_t,
                              void* stream);

/*
 * Gradients of the recurrence (reverse mode) for training: given the
 * forward inputs and the gradients dy of y (and optionally dh_final of the
 * final state), computes the gradients of
 *
 *   L = sum_t <y_t, dy_t> + <h_{T-1}, dh_final>
 *
 * with respect to every input: dx, dB, dC in the inputs' layouts, ddt,
 * dlam [batch, T, H], dtheta [batch, T, H, N/2], dA [H], all float32
 * whatever the storage type.  The recurrence is the one m3_prefill computes
 * (Mamba-3 paper summary, Proposition 1; explainer, "second improvement";
 * paper summary, item 3 for the rank R); the pages release training kernels
 * without describing them, so this is the plain adjoint of that recurrence:
 * with G_t = dL/dh_t, G_t = C_t dy_t^T + alpha_{t+1} R_{t+1}^T G_{t+1}, and
 * each token's gradients follow from h_t, h_{t-1} and G_t.
 *
 * With N = P = 64 (R of 1, 2 or 4) the gradients are taken by chunks of
 * L = 64 / R tokens with the contractions on the matrix cores (float32): a
 * local pass forms each chunk's state and adjoint contributions, a chain
 * pass composes them into every chunk's entry state and exit adjoint, a
 * gradient pass forms every token's gradients from its chunk's products,
 * and a final pass combines the per-token scalar partials.  The workspace
 * holds, per (batch, head), nC + 1 entry states and nC exit adjoints
 * (N x P float each, nC = ceil(T / L)), 65 floats per chunk and 16 bytes
 * per token (each area rounded up to 256 bytes).  Four kernel launches.
 * Other shapes with N * P <= 4096: the sequence is cut into segments of S
 * tokens (32, or 16 or 8 where the segment's staged inputs would not fit the
 * LDS): a
 * local pass walks every segment from a zero state both ways, a chain pass
 * composes the segments into each one's entry state and exit adjoint, and
 * a gradient pass recomputes each segment's states in blocks of 8 tokens
 * on chip and walks them backward.  The workspace holds two N x P float
 * states per segment-head, plus per segment a decay and N/2 angles, plus
 * 4 bytes per token-head (each area rounded up to 256 bytes).  Four kernel
 * launches.
 * With N * P = 8192 the states h_t and G_t of every token are materialised
 * in the workspace instead (8 N P bytes per token-head plus 4), so the call
 * moves about 5 x 4 N P bytes per token-head through HBM.  Four kernel
 * launches.
 * m3_backward_workspace_size gives the bytes for each case.  dy has x's
 * layout and storage type; dh_final, if given, is [batch, H, N, P] float.
 * lam and theta are required.  N must be 16, 32, 64, 128 or 256 with
 * N * P <= 8192; P and R as for m3_prefill.  x and dy need 16-byte
 * alignment, the other pointers element alignment and the workspace 256
 * bytes.  With batch * seqlen == 0 only dA is written (zeros).
 */
size_t m3_backward_workspace_size(const m3_dims* dims, m3_dtype dtype);

m3_status m3_backward(const m3_dims* dims, m3_dtype dtype, const void* x, const float* dt,
                      const float* A, const float* lam, const float* theta, const void* B,
                      const void* C, const void* dy, const float* dh_final, float* dx,
                      float* ddt, float* dA, float* dlam, float* dtheta, float* dB, float* dC,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block-side steps on either side of the SSM (Mamba-3 paper translation,
 * section 3.4 "Mamba-3 architecture"; paper summary, "Steps & Procedures"):
 * BCNorm -- an RMS normalisation after the B and C projections, in the
 * manner of QK normalisation -- then a learnable head-specific channel-wise
 * bias on B and C, and the MIMO projections of section 3.3, which take the
 * input from P to P x R channels and the output back, with additive
 * parameter growth.  The pages leave the projections' exact form to an
 * appendix they do not include; read here as per-head, per-rank
 * channel-wise scalings (2 R P parameters per head):
 *
 *   m3_block_prepass:   B~[r] = B[r] / sqrt(mean_n B[r]^2 + eps) * norm_B[h] + bias_B[h][r]
 *                       C~[r] likewise with norm_C, bias_C
 *                       X[r]  = x * up[h][r]
 *   m3_block_postpass:  y_out = sum_r down[h][r] * y[r]
 *
 * per token and head (mean over the N channels of the row).  The pre-pass's
 * outputs are the x, B, C of m3_prefill / m3_decode_step; the post-pass
 * takes their y.
 *
 * Layouts (row-major, dense; T the storage type of dtype; dims->seqlen may
 * be 1 for a decode token):
 *   x, y_out              [batch, T, H, P]
 *   B, C, B~, C~          [batch, T, H, R, N]
 *   X, y                  [batch, T, H, R, P]
 *   norm_B, norm_C        [H, N]      float
 *   bias_B, bias_C        [H, R, N]   float
 *   up, down              [H, R, P]   float
 * N must be 16, 32, 64, 128 or 256; P and R as for m3_prefill.  Every
 * array (x, B, C, X, B~, C~, y, y_out and the weights) needs 16-byte
 * alignment.
 * B~ may be B and C~ may be C (in place), X may be x when R = 1; other
 * overlaps between inputs and outputs are not allowed.  eps >= 0 (finite).
 * One kernel launch each; batch * seqlen == 0 enqueues nothing.
 */
m3_status m3_block_prepass(const m3_dims* dims, m3_dtype dtype, const void* x, const void* B,
                           const void* C, const float* norm_B, const float* norm_C,
                           const float* bias_B, const float* bias_C, const float* up, float eps,
                           void* x_out, void* B_out, void* C_out, void* stream);

m3_status m3_block_postpass(const m3_dims* dims, m3_dtype dtype, const void* y,
                            const float* down, void* y_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* M3SSM_H_ */
