"""fp64 CPU oracle for the Mamba-3 SSM layer recurrence.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The GPU
library (``state_space_sequence_exp_amd``) never imports it, and this package
imports nothing from the GPU library.

Two independent formulations live here:

* ``prefill`` / ``decode_step`` -- the sequential complex-valued recurrence,
  written in C (``m3_oracle.c``), fp64, threaded over (batch, head) units.
  It follows Proposition 1 of the Mamba-3 paper summary (aipaper.cc,
  "Mathematical formulas and key details", item 1) with the complex
  transition of the explainer (yunpan.plus, "second improvement").
* ``bruteforce.masked_form`` -- the parallel (structured-mask) form, written
  in NumPy for short sequences: rotated B, C (Proposition 3 of the paper
  summary) and the mask = decay matrix x 2-band matrix (Mamba-3 paper, P1
  section 3.1, equation 7 and Remark 5).

Every function here is pinned in ``tests/test_oracle_pins.py`` against
closed forms, special cases and the masked form.  No function is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "m3_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``m3_oracle.c`` into ``liboracle.so`` with gcc (host only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        i64p = ctypes.POINTER(ctypes.c_int64)
        fp = ctypes.c_void_p
        lib.m3o_prefill.restype = ctypes.c_int
        lib.m3o_prefill.argtypes = [i64p, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                                    i64p, ctypes.c_int64, ctypes.c_int]
        lib.m3o_decode_step.restype = ctypes.c_int
        lib.m3o_decode_step.argtypes = [i64p, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                                        fp, i64p, ctypes.c_int64, ctypes.c_int]
        _lib = lib
    return _lib


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _units(units, total):
    if units is None:
        return None, total
    u = np.ascontiguousarray(np.asarray(units, dtype=np.int64))
    return u, int(u.size)


def prefill(x, dt, A, lam, theta, B, C, *, h0=None, x_halo=None, B_halo=None,
            units: Optional[Sequence[int]] = None, nthreads: int = 0,
            want_y: bool = True):
    """Sequential fp64 recurrence over a whole sequence.

    Shapes: x [Bt,T,H,R,P]; B, C [Bt,T,H,R,N]; dt, lam [Bt,T,H];
    theta [Bt,T,H,N/2]; A [H]; optional h0 [Bt,H,N,P], x_halo [Bt,H,R,P],
    B_halo [Bt,H,R,N] (the state and the previous token's input before the
    first token).  Returns (y [Bt,T,H,R,P] float64, h_final [Bt,H,N,P]
    float64).  With ``units`` (ids b*H+h) only those units are computed; the
    other entries of y and h_final are NaN.
    """
    x, dt, A, lam, theta, B, C = map(_f32, (x, dt, A, lam, theta, B, C))
    nb, nt, nh, nr, npd = x.shape
    nn = B.shape[-1]
    assert B.shape == (nb, nt, nh, nr, nn) and C.shape == B.shape
    assert dt.shape == (nb, nt, nh) and lam.shape == dt.shape
    assert theta.shape == (nb, nt, nh, nn // 2) and A.shape == (nh,)
    h0a = None if h0 is None else np.ascontiguousarray(np.asarray(h0, dtype=np.float64))
    if h0a is not None:
        assert h0a.shape == (nb, nh, nn, npd)
    xh = None if x_halo is None else _f32(x_halo)
    bh = None if B_halo is None else _f32(B_halo)
    if xh is not None:
        assert xh.shape == (nb, nh, nr, npd) and bh is not None and bh.shape == (nb, nh, nr, nn)
    y = np.full((nb, nt, nh, nr, npd), np.nan) if want_y else None
    hf = np.full((nb, nh, nn, npd), np.nan)
    u, nu = _units(units, nb * nh)
    dims = (ctypes.c_int64 * 6)(nb, nt, nh, npd, nn, nr)
    rc = _load().m3o_prefill(dims, _ptr(x), _ptr(dt), _ptr(A), _ptr(lam), _ptr(theta),
                             _ptr(B), _ptr(C), _ptr(h0a), _ptr(xh), _ptr(bh), _ptr(y),
                             _ptr(hf),
                             None if u is None else u.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                             nu, int(nthreads))
    if rc != 0:
        raise RuntimeError("m3o_prefill failed with code %d" % rc)
    return y, hf


def decode_step(h, x_t, x_prev, B_t, B_prev, C_t, dt, A, lam, theta, *,
                units: Optional[Sequence[int]] = None, nthreads: int = 0):
    """One fp64 decode step.  h [S,H,N,P] (float64); x_t, x_prev [S,H,R,P];
    B_t, B_prev, C_t [S,H,R,N]; dt, lam [S,H]; theta [S,H,N/2]; A [H].
    Returns (y [S,H,R,P], h_new [S,H,N,P]) as float64.  With ``units`` only
    those (s*H+h) units are computed; other entries are NaN."""
    h = np.ascontiguousarray(np.asarray(h, dtype=np.float64))
    x_t, x_prev, B_t, B_prev, C_t, dt, A, lam, theta = map(
        _f32, (x_t, x_prev, B_t, B_prev, C_t, dt, A, lam, theta))
    ns, nh, nn, npd = h.shape
    nr = x_t.shape[2]
    assert x_t.shape == (ns, nh, nr, npd) and x_prev.shape == x_t.shape
    assert B_t.shape == (ns, nh, nr, nn) and B_prev.shape == B_t.shape and C_t.shape == B_t.shape
    assert dt.shape == (ns, nh) and lam.shape == dt.shape and A.shape == (nh,)
    assert theta.shape == (ns, nh, nn // 2)
    y = np.full((ns, nh, nr, npd), np.nan)
    h_new = np.full_like(h, np.nan)
    u, nu = _units(units, ns * nh)
    dims = (ctypes.c_int64 * 6)(ns, 1, nh, npd, nn, nr)
    rc = _load().m3o_decode_step(dims, _ptr(h), _ptr(x_t), _ptr(x_prev), _ptr(B_t),
                                 _ptr(B_prev), _ptr(C_t), _ptr(dt), _ptr(A), _ptr(lam),
                                 _ptr(theta), _ptr(y), _ptr(h_new),
                                 None if u is None else u.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                 nu, int(nthreads))
    if rc != 0:
        raise RuntimeError("m3o_decode_step failed with code %d" % rc)
    return y, h_new


def n_threads() -> int:
    """Threads the oracle uses by default (online processors)."""
    return os.cpu_count() or 1
