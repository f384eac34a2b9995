"""ctypes binding of libm3ssm (include/m3ssm.h).

Argument marshalling only: every step of the recurrence runs in the HIP
kernels of libm3ssm.so.  PyTorch supplies device memory and the current
stream.  If the library is not built this module raises on first use; there
is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libm3ssm.so")

M3_SUCCESS = 0
M3_ERR_INVALID_VALUE = 1
M3_ERR_NOT_SUPPORTED = 2
M3_ERR_WORKSPACE = 3
M3_ERR_HIP = 4
M3_ERR_CHAIN = 5
M3_F32 = 0
M3_BF16 = 1

# every function declared in include/m3ssm.h
ABI_SYMBOLS = ("m3_version", "m3_status_string", "m3_prefill_workspace_size", "m3_prefill",
               "m3_prefill_workspace_error", "m3_prefill_noalloc", "m3_prefill_from_state", "m3_decode_step", "m3_decode_step_mfma", "m3_block_prepass", "m3_block_postpass",
               "m3_backward_workspace_size", "m3_backward")


class M3Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s" % (where, status_string(status)))


class M3Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim_p", ctypes.c_int64),
                ("dstate_n", ctypes.c_int64), ("rank_r", ctypes.c_int64)]


_lib = None


def load_library(path: Optional[str] = None):
    """Load libm3ssm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libm3ssm.so not found at %s; build it with "
                           "`python -m state_space_sequence_exp_amd.build`" % p)
    # torch first: it brings its own HIP runtime, and the library must bind
    # to the same one (loaded before torch, the library would start the
    # system runtime, which then sees no device next to torch's)
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    vp = ctypes.c_void_p
    dp = ctypes.POINTER(M3Dims)
    lib.m3_version.restype = ctypes.c_int
    lib.m3_version.argtypes = []
    lib.m3_status_string.restype = ctypes.c_char_p
    lib.m3_status_string.argtypes = [ctypes.c_int]
    lib.m3_prefill_workspace_size.restype = ctypes.c_size_t
    lib.m3_prefill_workspace_size.argtypes = [dp, ctypes.c_int, ctypes.c_int]
    lib.m3_prefill.restype = ctypes.c_int
    lib.m3_prefill.argtypes = [dp, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp,
                               vp, vp, ctypes.c_size_t, vp]
    lib.m3_prefill_workspace_error.restype = ctypes.c_int
    lib.m3_prefill_workspace_error.argtypes = [vp, ctypes.c_size_t, ctypes.c_int,
                                               ctypes.POINTER(ctypes.c_int), vp]
    lib.m3_prefill_noalloc.restype = ctypes.c_int
    lib.m3_prefill_noalloc.argtypes = [dp, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp,
                                       vp, vp, vp, vp]
    lib.m3_prefill_from_state.restype = ctypes.c_int
    lib.m3_prefill_from_state.argtypes = [dp, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp,
                                          vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.m3_decode_step.restype = ctypes.c_int
    lib.m3_decode_step.argtypes = [dp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   vp, vp]
    lib.m3_decode_step_mfma.restype = ctypes.c_int
    lib.m3_decode_step_mfma.argtypes = [dp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   vp, vp]
    lib.m3_backward_workspace_size.restype = ctypes.c_size_t
    lib.m3_backward_workspace_size.argtypes = [dp, ctypes.c_int]
    lib.m3_backward.restype = ctypes.c_int
    lib.m3_backward.argtypes = [dp, ctypes.c_int] + [vp] * 17 + [ctypes.c_size_t, vp]
    lib.m3_block_prepass.restype = ctypes.c_int
    lib.m3_block_prepass.argtypes = [dp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp,
                                     ctypes.c_float, vp, vp, vp, vp]
    lib.m3_block_postpass.restype = ctypes.c_int
    lib.m3_block_postpass.argtypes = [dp, ctypes.c_int, vp, vp, vp, vp]
    if path is None:
        _lib = lib
    return lib


def version() -> int:
    return load_library().m3_version()


def status_string(status: int) -> str:
    return load_library().m3_status_string(int(status)).decode()


def _dims(batch, seqlen, nheads, P, N, R) -> M3Dims:
    return M3Dims(int(batch), int(seqlen), int(nheads), int(P), int(N), int(R))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return M3_F32
    if t.dtype == torch.bfloat16:
        return M3_BF16
    raise TypeError("x, B, C must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.device != device:
        raise ValueError("%s: on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def prefill_workspace_size(batch, seqlen, nheads, P, N, R, chunk, dtype) -> int:
    """Bytes of workspace m3_prefill needs (0: nothing to do, or unsupported)."""
    import torch
    code = dtype if isinstance(dtype, int) else (M3_BF16 if dtype == torch.bfloat16 else M3_F32)
    d = _dims(batch, seqlen, nheads, P, N, R)
    return int(load_library().m3_prefill_workspace_size(ctypes.byref(d), int(chunk), code))


def prefill_workspace_error(workspace, *, clear: bool = False, stream=None) -> int:
    """The error word of a prefill workspace once the stream's work has
    finished (m3_prefill_workspace_error; synchronises the stream): 0 when
    every chain wait completed, 1 after a timed-out wait (outputs NaN), 2
    after dirty counters.  With clear=True a nonzero word is reset."""
    word = ctypes.c_int(0)
    nbytes = workspace.numel() * workspace.element_size()
    st = load_library().m3_prefill_workspace_error(_ptr(workspace), nbytes, int(bool(clear)),
                                                   ctypes.byref(word), _stream(stream))
    if st not in (M3_SUCCESS, M3_ERR_CHAIN):
        raise M3Error(st, "m3_prefill_workspace_error")
    return int(word.value)


def prefill(x, dt, A, lam, theta, B, C, chunk: int, *, h0=None, x_prev=None, B_prev=None,
            y=None, h_final=None, want_h_final: bool = True, workspace=None,
            check: bool = False, stream=None) -> Tuple:
    """Chunked prefill on the GPU.

    x [Bt,T,H,R,P] (or [Bt,T,H,P] for R=1); B, C [Bt,T,H,R,N] (or [Bt,T,H,N]);
    dt, lam [Bt,T,H]; theta [Bt,T,H,N/2]; A [H].  x, B, C float32 or
    bfloat16 (same dtype), the rest float32, all contiguous on one GPU.
    lam=None gives the exponential-Euler rule (lam = 1, Mamba-2's
    discretisation) and theta=None a real state (no rotation).
    To continue a sequence pass h0 [Bt,H,N,P] float32 (the state before the
    first token) and/or x_prev [Bt,H,R,P] with B_prev [Bt,H,R,N] (the
    previous token's x and B, x's dtype; R axis optional for R=1); this calls
    m3_prefill_from_state.  h_final may be h0 (in-place update).
    check=True synchronises the stream after the call and raises M3Error
    (M3_ERR_CHAIN) if the workspace's error word is set.
    Returns (y with x's shape and dtype, h_final [Bt,H,N,P] float32 or None).
    """
    import torch
    lib = load_library()
    squeeze = x.dim() == 4
    x5 = x.unsqueeze(3) if squeeze else x
    B5 = B.unsqueeze(3) if B.dim() == 4 else B
    C5 = C.unsqueeze(3) if C.dim() == 4 else C
    nb, nt, nh, nr, npd = x5.shape
    nn = B5.shape[-1]
    dev = x.device
    code = _dtype_code(x)
    _check(x5, "x", x.dtype, (nb, nt, nh, nr, npd), dev)
    _check(B5, "B", x.dtype, (nb, nt, nh, nr, nn), dev)
    _check(C5, "C", x.dtype, (nb, nt, nh, nr, nn), dev)
    _check(dt, "dt", torch.float32, (nb, nt, nh), dev)
    if lam is not None:
        _check(lam, "lam", torch.float32, (nb, nt, nh), dev)
    if theta is not None:
        _check(theta, "theta", torch.float32, (nb, nt, nh, nn // 2), dev)
    _check(A, "A", torch.float32, (nh,), dev)
    if y is None:
        y = torch.empty_like(x)
    else:
        _check(y, "y", x.dtype, tuple(x.shape), dev)
    if h_final is None and want_h_final:
        h_final = torch.empty((nb, nh, nn, npd), dtype=torch.float32, device=dev)
    elif h_final is not None:
        _check(h_final, "h_final", torch.float32, (nb, nh, nn, npd), dev)
    cont = h0 is not None or x_prev is not None or B_prev is not None
    if h0 is not None:
        _check(h0, "h0", torch.float32, (nb, nh, nn, npd), dev)
    if (x_prev is None) != (B_prev is None):
        raise ValueError("x_prev and B_prev go together")
    if x_prev is not None:
        x_prev = x_prev.unsqueeze(2) if x_prev.dim() == 3 else x_prev
        B_prev = B_prev.unsqueeze(2) if B_prev.dim() == 3 else B_prev
        _check(x_prev, "x_prev", x.dtype, (nb, nh, nr, npd), dev)
        _check(B_prev, "B_prev", x.dtype, (nb, nh, nr, nn), dev)
    d = _dims(nb, nt, nh, npd, nn, nr)
    need = int(lib.m3_prefill_workspace_size(ctypes.byref(d), int(chunk), code))
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if cont:
        st = lib.m3_prefill_from_state(ctypes.byref(d), code, int(chunk), _ptr(h0), _ptr(x_prev),
                                       _ptr(B_prev), _ptr(x5), _ptr(dt), _ptr(A), _ptr(lam),
                                       _ptr(theta), _ptr(B5), _ptr(C5), _ptr(y), _ptr(h_final),
                                       _ptr(workspace), ws_bytes, _stream(stream))
    else:
        st = lib.m3_prefill(ctypes.byref(d), code, int(chunk), _ptr(x5), _ptr(dt), _ptr(A),
                            _ptr(lam), _ptr(theta), _ptr(B5), _ptr(C5), _ptr(y), _ptr(h_final),
                            _ptr(workspace), ws_bytes, _stream(stream))
    if st != M3_SUCCESS:
        raise M3Error(st, "m3_prefill_from_state" if cont else "m3_prefill")
    if check and workspace is not None:
        if prefill_workspace_error(workspace, stream=stream) != 0:
            raise M3Error(M3_ERR_CHAIN, "m3_prefill_from_state" if cont else "m3_prefill")
    return y, h_final


# device scratch of m3_prefill_noalloc, per GPU (M3_PREFILL_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20


def prefill_noalloc(x, dt, A, lam, theta, B, C, chunk: int, y, h_final=None,
                    stream=None) -> Tuple:
    """Chunked prefill through m3_prefill_noalloc: no workspace, and nothing
    allocated by this call (y, and h_final if wanted, are the caller's).  The
    library's per-GPU scratch stands in for the workspace, so calls that
    overlap on one GPU race.  Shapes as for prefill()."""
    import torch
    lib = load_library()
    x5 = x.unsqueeze(3) if x.dim() == 4 else x
    B5 = B.unsqueeze(3) if B.dim() == 4 else B
    C5 = C.unsqueeze(3) if C.dim() == 4 else C
    nb, nt, nh, nr, npd = x5.shape
    nn = B5.shape[-1]
    dev = x.device
    code = _dtype_code(x)
    _check(x5, "x", x.dtype, (nb, nt, nh, nr, npd), dev)
    _check(B5, "B", x.dtype, (nb, nt, nh, nr, nn), dev)
    _check(C5, "C", x.dtype, (nb, nt, nh, nr, nn), dev)
    _check(dt, "dt", torch.float32, (nb, nt, nh), dev)
    if lam is not None:
        _check(lam, "lam", torch.float32, (nb, nt, nh), dev)
    if theta is not None:
        _check(theta, "theta", torch.float32, (nb, nt, nh, nn // 2), dev)
    _check(A, "A", torch.float32, (nh,), dev)
    _check(y, "y", x.dtype, tuple(x.shape), dev)
    if h_final is not None:
        _check(h_final, "h_final", torch.float32, (nb, nh, nn, npd), dev)
    d = _dims(nb, nt, nh, npd, nn, nr)
    st = lib.m3_prefill_noalloc(ctypes.byref(d), code, int(chunk), _ptr(x5), _ptr(dt), _ptr(A),
                                _ptr(lam), _ptr(theta), _ptr(B5), _ptr(C5), _ptr(y),
                                _ptr(h_final), _stream(stream))
    if st != M3_SUCCESS:
        raise M3Error(st, "m3_prefill_noalloc")
    return y, h_final


def decode_step(h, x_t, x_prev, B_t, B_prev, C_t, dt, A, lam, theta, *, h_out=None, y=None,
                stream=None, matrix_cores: bool = False) -> Tuple:
    """One decode step on the GPU.

    h [S,H,N,P] float32; x_t, x_prev [S,H,R,P]; B_t, B_prev, C_t [S,H,R,N]
    (float32 or bfloat16); dt, lam [S,H]; theta [S,H,N/2]; A [H].
    lam=None gives the exponential-Euler rule (lam = 1; x_prev and B_prev
    are then not read and may be None) and theta=None a real state.
    h_out defaults to h itself (in-place update).  Returns (y_t [S,H,R,P],
    h_out).  matrix_cores=True calls m3_decode_step_mfma (the rank-2R
    update on MFMA; R 2 or 4, P 64, N a multiple of 16 up to 128).
    """
    import torch
    lib = load_library()
    ns, nh, nn, npd = h.shape
    nr = x_t.shape[2]
    dev = h.device
    code = _dtype_code(x_t)
    _check(h, "h", torch.float32, (ns, nh, nn, npd), dev)
    if lam is None and x_prev is None and B_prev is None:
        x_prev = B_prev = None
    elif x_prev is None or B_prev is None:
        raise ValueError("x_prev and B_prev are required with lam")
    for name, t in (("x_t", x_t), ("x_prev", x_prev)):
        if t is not None:
            _check(t, name, x_t.dtype, (ns, nh, nr, npd), dev)
    for name, t in (("B_t", B_t), ("B_prev", B_prev), ("C_t", C_t)):
        if t is not None:
            _check(t, name, x_t.dtype, (ns, nh, nr, nn), dev)
    _check(dt, "dt", torch.float32, (ns, nh), dev)
    if lam is not None:
        _check(lam, "lam", torch.float32, (ns, nh), dev)
    if theta is not None:
        _check(theta, "theta", torch.float32, (ns, nh, nn // 2), dev)
    _check(A, "A", torch.float32, (nh,), dev)
    if h_out is None:
        h_out = h
    else:
        _check(h_out, "h_out", torch.float32, (ns, nh, nn, npd), dev)
    if y is None:
        y = torch.empty((ns, nh, nr, npd), dtype=x_t.dtype, device=dev)
    else:
        _check(y, "y", x_t.dtype, (ns, nh, nr, npd), dev)
    d = _dims(ns, 1, nh, npd, nn, nr)
    fn = lib.m3_decode_step_mfma if matrix_cores else lib.m3_decode_step
    st = fn(ctypes.byref(d), code, _ptr(h), _ptr(h_out), _ptr(x_t), _ptr(x_prev), _ptr(B_t),
            _ptr(B_prev), _ptr(C_t), _ptr(dt), _ptr(A), _ptr(lam), _ptr(theta), _ptr(y),
            _stream(stream))
    if st != M3_SUCCESS:
        raise M3Error(st, "m3_decode_step_mfma" if matrix_cores else "m3_decode_step")
    return y, h_out


def block_prepass(x, B, C, norm_B, norm_C, bias_B, bias_C, up, eps: float = 1e-6, *,
                  x_out=None, B_out=None, C_out=None, stream=None) -> Tuple:
    """BCNorm + bias on B and C, MIMO up-projection of x (m3_block_prepass).

    x [Bt,T,H,P]; B, C [Bt,T,H,R,N] (float32 or bfloat16, same dtype);
    norm_B, norm_C [H,N]; bias_B, bias_C [H,R,N]; up [H,R,P] float32.
    Returns (X [Bt,T,H,R,P], B~, C~ [Bt,T,H,R,N]) in x's dtype.
    """
    import torch
    lib = load_library()
    nb, nt, nh, npd = x.shape
    nr, nn = B.shape[3], B.shape[4]
    dev = x.device
    code = _dtype_code(x)
    _check(x, "x", x.dtype, (nb, nt, nh, npd), dev)
    _check(B, "B", x.dtype, (nb, nt, nh, nr, nn), dev)
    _check(C, "C", x.dtype, (nb, nt, nh, nr, nn), dev)
    _check(norm_B, "norm_B", torch.float32, (nh, nn), dev)
    _check(norm_C, "norm_C", torch.float32, (nh, nn), dev)
    _check(bias_B, "bias_B", torch.float32, (nh, nr, nn), dev)
    _check(bias_C, "bias_C", torch.float32, (nh, nr, nn), dev)
    _check(up, "up", torch.float32, (nh, nr, npd), dev)
    if x_out is None:
        x_out = torch.empty((nb, nt, nh, nr, npd), dtype=x.dtype, device=dev)
    if B_out is None:
        B_out = torch.empty_like(B)
    if C_out is None:
        C_out = torch.empty_like(C)
    _check(x_out, "x_out", x.dtype, (nb, nt, nh, nr, npd), dev)
    _check(B_out, "B_out", x.dtype, tuple(B.shape), dev)
    _check(C_out, "C_out", x.dtype, tuple(C.shape), dev)
    d = _dims(nb, nt, nh, npd, nn, nr)
    st = lib.m3_block_prepass(ctypes.byref(d), code, _ptr(x), _ptr(B), _ptr(C), _ptr(norm_B),
                              _ptr(norm_C), _ptr(bias_B), _ptr(bias_C), _ptr(up),
                              ctypes.c_float(eps), _ptr(x_out), _ptr(B_out), _ptr(C_out),
                              _stream(stream))
    if st != M3_SUCCESS:
        raise M3Error(st, "m3_block_prepass")
    return x_out, B_out, C_out


def block_postpass(y, down, *, y_out=None, stream=None):
    """MIMO down-projection y_out = sum_r down[h,r] * y[r] (m3_block_postpass).

    y [Bt,T,H,R,P] float32 or bfloat16; down [H,R,P] float32.
    Returns y_out [Bt,T,H,P] in y's dtype.
    """
    import torch
    lib = load_library()
    nb, nt, nh, nr, npd = y.shape
    dev = y.device
    code = _dtype_code(y)
    _check(y, "y", y.dtype, (nb, nt, nh, nr, npd), dev)
    _check(down, "down", torch.float32, (nh, nr, npd), dev)
    if y_out is None:
        y_out = torch.empty((nb, nt, nh, npd), dtype=y.dtype, device=dev)
    _check(y_out, "y_out", y.dtype, (nb, nt, nh, npd), dev)
    # the state size does not enter the post-pass; any supported value
    d = _dims(nb, nt, nh, npd, 64, nr)
    st = lib.m3_block_postpass(ctypes.byref(d), code, _ptr(y), _ptr(down), _ptr(y_out),
                               _stream(stream))
    if st != M3_SUCCESS:
        raise M3Error(st, "m3_block_postpass")
    return y_out


def backward_workspace_size(batch, seqlen, nheads, P, N, R, dtype) -> int:
    """Bytes of workspace m3_backward needs (0: nothing to do, or unsupported)."""
    import torch
    code = dtype if isinstance(dtype, int) else (M3_BF16 if dtype == torch.bfloat16 else M3_F32)
    d = _dims(batch, seqlen, nheads, P, N, R)
    return int(load_library().m3_backward_workspace_size(ctypes.byref(d), code))


def backward(x, dt, A, lam, theta, B, C, dy, *, dh_final=None, workspace=None, stream=None):
    """Gradients of sum(y * dy) (+ sum(h_final * dh_final)) for the prefill
    inputs (m3_backward).  Shapes as for prefill; dy has x's shape and dtype.
    Returns a dict of float32 gradients: x, dt, A, lam, theta, B, C."""
    import torch
    lib = load_library()
    squeeze = x.dim() == 4
    x5 = x.unsqueeze(3) if squeeze else x
    B5 = B.unsqueeze(3) if B.dim() == 4 else B
    C5 = C.unsqueeze(3) if C.dim() == 4 else C
    dy5 = dy.unsqueeze(3) if dy.dim() == 4 else dy
    nb, nt, nh, nr, npd = x5.shape
    nn = B5.shape[-1]
    dev = x.device
    code = _dtype_code(x)
    _check(x5, "x", x.dtype, (nb, nt, nh, nr, npd), dev)
    _check(dy5, "dy", x.dtype, (nb, nt, nh, nr, npd), dev)
    _check(B5, "B", x.dtype, (nb, nt, nh, nr, nn), dev)
    _check(C5, "C", x.dtype, (nb, nt, nh, nr, nn), dev)
    _check(dt, "dt", torch.float32, (nb, nt, nh), dev)
    _check(lam, "lam", torch.float32, (nb, nt, nh), dev)
    _check(theta, "theta", torch.float32, (nb, nt, nh, nn // 2), dev)
    _check(A, "A", torch.float32, (nh,), dev)
    if dh_final is not None:
        _check(dh_final, "dh_final", torch.float32, (nb, nh, nn, npd), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"x": torch.empty((nb, nt, nh, nr, npd), **f32), "dt": torch.empty((nb, nt, nh), **f32),
         "A": torch.empty((nh,), **f32), "lam": torch.empty((nb, nt, nh), **f32),
         "theta": torch.empty((nb, nt, nh, nn // 2), **f32),
         "B": torch.empty((nb, nt, nh, nr, nn), **f32), "C": torch.empty((nb, nt, nh, nr, nn), **f32)}
    d = _dims(nb, nt, nh, npd, nn, nr)
    need = int(lib.m3_backward_workspace_size(ctypes.byref(d), code))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.m3_backward(ctypes.byref(d), code, _ptr(x5), _ptr(dt), _ptr(A), _ptr(lam),
                         _ptr(theta), _ptr(B5), _ptr(C5), _ptr(dy5), _ptr(dh_final),
                         _ptr(g["x"]), _ptr(g["dt"]), _ptr(g["A"]), _ptr(g["lam"]),
                         _ptr(g["theta"]), _ptr(g["B"]), _ptr(g["C"]), _ptr(workspace),
                         ws_bytes, _stream(stream))
    if st != M3_SUCCESS:
        raise M3Error(st, "m3_backward")
    if squeeze:
        g["x"] = g["x"].squeeze(3)
    return g
