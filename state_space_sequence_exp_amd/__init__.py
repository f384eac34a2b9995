"""libm3ssm: the Mamba-3 SSM layer recurrence (exponential-trapezoidal
discretisation, complex state as a data-dependent RoPE, rank-R MIMO) as
hand-written HIP kernels for AMD Instinct MI355X (gfx950), behind a C ABI
(include/m3ssm.h).

Python entry points (ctypes; PyTorch tensors supply device memory and the
current stream):

    prefill(x, dt, A, lam, theta, B, C, chunk[, h0, x_prev, B_prev]) -> (y, h_final)
    prefill_noalloc(x, dt, A, lam, theta, B, C, chunk, y[, h_final])   (no workspace)
    decode_step(h, x_t, x_prev, B_t, B_prev, C_t, dt, A, lam, theta) -> (y_t, h)
    block_prepass(x, B, C, norm_B, norm_C, bias_B, bias_C, up, eps) -> (X, B~, C~)
    block_postpass(y, down) -> y_out
    backward(x, dt, A, lam, theta, B, C, dy[, dh_final]) -> dict of gradients
    prefill_workspace_size(...), prefill_workspace_error(workspace), version(),
    status_string(code)

``inputs`` draws the seeded synthetic workloads.  Build the library with
``python -m state_space_sequence_exp_amd.build``.
"""
from ._binding import (ABI_SYMBOLS, LIB_PATH, M3_BF16, M3_ERR_CHAIN, M3_ERR_HIP,
                       M3_ERR_INVALID_VALUE, M3_ERR_NOT_SUPPORTED, M3_ERR_WORKSPACE, M3_F32,
                       M3_SUCCESS, M3Dims, M3Error, backward, backward_workspace_size,
                       block_postpass, block_prepass, decode_step, load_library, prefill,
                       prefill_noalloc, prefill_workspace_error, prefill_workspace_size,
                       status_string, version)

__all__ = ["prefill", "prefill_noalloc", "decode_step", "block_prepass", "block_postpass", "backward",
           "backward_workspace_size", "prefill_workspace_size", "prefill_workspace_error",
           "version", "status_string",
           "load_library", "M3Error", "M3Dims", "ABI_SYMBOLS", "LIB_PATH", "M3_SUCCESS",
           "M3_ERR_INVALID_VALUE", "M3_ERR_NOT_SUPPORTED", "M3_ERR_WORKSPACE", "M3_ERR_HIP",
           "M3_ERR_CHAIN",
           "M3_F32", "M3_BF16"]
