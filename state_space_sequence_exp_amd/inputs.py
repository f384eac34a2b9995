"""Seeded synthetic inputs for the Mamba-3 SSM layer recurrence.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the recurrence's arithmetic, so both the GPU path and the
CPU oracle may consume what it produces.

Recipe (per configuration, NumPy PCG64 seeded with the given seed; draws in
this fixed order):

    A      = -exp(U(a_lo, a_hi))      [H]            (default U(-2, 0))
    dt     = softplus(N(0,1) - 1)     [B,T,H]
    lam    = sigmoid(N(0,1))          [B,T,H]
    theta  = U(-pi, pi)               [B,T,H,N/2]
    x      = N(0,1)                   [B,T,H,R,P]
    B      = N(0, 1/N)                [B,T,H,R,N]
    C      = N(0, 1/N)                [B,T,H,R,N]

A, dt, lam are drawn in float64 and rounded to float32; theta, x, B, C are
drawn directly in float32 (cheaper at 10^8 elements).  For bf16
configurations x, B and C are then rounded to bfloat16 (round to nearest
even) and the returned float32 arrays hold exactly those bfloat16 values.

The five workloads are shaped like the Mamba-3 pages' 1.5B-scale layers
(d_model 2048, d_inner 4096 = 64 heads x 64), their 16K-token latency run
and their batch-128-class decode benchmark; the trained weights and the
text corpus those pages use are not available, and these random inputs
stand in for them.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    batch: int
    seqlen: int
    nheads: int
    N: int
    P: int
    R: int
    dtype: str      # "f32" or "bf16": storage type of x, B, C and y
    chunk: int


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int      # sequences
    nheads: int
    N: int
    P: int
    R: int
    dtype: str
    steps: int
    ring: int       # distinct per-step input sets cycled through


WORKLOADS = {
    0: PrefillConfig("tiny_siso_fp32_b1_h1_t256_n16_p16", 1, 256, 1, 16, 16, 1, "f32", 32),
    1: PrefillConfig("siso_prefill_b4_t2048_h16_n64_p64", 4, 2048, 16, 64, 64, 1, "bf16", 64),
    2: PrefillConfig("mimo_r4_prefill_b4_t4096_h16_n64_p64", 4, 4096, 16, 64, 64, 4, "bf16", 64),
    3: PrefillConfig("long_siso_prefill_b1_t16384_h64_n128_p64", 1, 16384, 64, 128, 64, 1, "bf16", 64),
    4: DecodeConfig("decode_mimo_r4_s256_h32_n128_p64", 256, 32, 128, 64, 4, "bf16", 1000, 16),
}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        rounded[nan] = 0x7FC0
    return rounded


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits (uint16) to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(a32: np.ndarray, dtype: str):
    """Return (float32 values as stored, raw storage array)."""
    if dtype == "f32":
        return a32, a32
    if dtype == "bf16":
        bits = bf16_round(a32)
        return bf16_to_f32(bits), bits
    raise ValueError("dtype must be 'f32' or 'bf16'")


def _softplus(v):
    return np.logaddexp(0.0, v)


def _sigmoid(v):
    return 0.5 * (1.0 + np.tanh(0.5 * v))


def prefill_inputs(batch: int, seqlen: int, nheads: int, N: int, P: int, R: int,
                   dtype: str, seed: int, a_range=(-2.0, 0.0)) -> Dict[str, np.ndarray]:
    """Draw one prefill problem.  Returned dict:

    x, B, C        float32 arrays holding the stored values ([B,T,H,R,P] / [B,T,H,R,N])
    x_raw, B_raw, C_raw   storage arrays (float32, or uint16 bfloat16 bits)
    dt, lam        float32 [B,T,H];  theta float32 [B,T,H,N/2];  A float32 [H]
    """
    if N % 2:
        raise ValueError("N must be even")
    rng = np.random.default_rng(seed)
    A = (-np.exp(rng.uniform(a_range[0], a_range[1], size=nheads))).astype(np.float32)
    dt = _softplus(rng.standard_normal((batch, seqlen, nheads)) - 1.0).astype(np.float32)
    lam = _sigmoid(rng.standard_normal((batch, seqlen, nheads))).astype(np.float32)
    theta = rng.uniform(-np.pi, np.pi, size=(batch, seqlen, nheads, N // 2)).astype(np.float32)
    x32 = rng.standard_normal((batch, seqlen, nheads, R, P), dtype=np.float32)
    B32 = rng.standard_normal((batch, seqlen, nheads, R, N), dtype=np.float32)
    B32 *= np.float32(1.0 / np.sqrt(N))
    C32 = rng.standard_normal((batch, seqlen, nheads, R, N), dtype=np.float32)
    C32 *= np.float32(1.0 / np.sqrt(N))
    x, x_raw = _store(x32, dtype)
    Bv, B_raw = _store(B32, dtype)
    Cv, C_raw = _store(C32, dtype)
    return dict(x=x, B=Bv, C=Cv, x_raw=x_raw, B_raw=B_raw, C_raw=C_raw,
                dt=dt, lam=lam, theta=theta, A=A, dtype=dtype)


def config_inputs(index: int, seed: Optional[int] = None, **overrides) -> Dict[str, np.ndarray]:
    """Inputs of prefill configuration ``index`` (0..3); seed defaults to the index."""
    cfg = WORKLOADS[index]
    if not isinstance(cfg, PrefillConfig):
        raise ValueError("configuration %d is not a prefill configuration" % index)
    kw = dict(batch=cfg.batch, seqlen=cfg.seqlen, nheads=cfg.nheads, N=cfg.N, P=cfg.P,
              R=cfg.R, dtype=cfg.dtype, seed=index if seed is None else seed)
    kw.update(overrides)
    return prefill_inputs(**kw)


def decode_inputs(batch: int, nheads: int, N: int, P: int, R: int, dtype: str, ring: int,
                  seed: int, a_range=(-2.0, 0.0)) -> Dict[str, np.ndarray]:
    """A ring of ``ring`` per-step input sets plus a random initial state.

    Returned dict: A [H]; h0 float32 [S,H,N,P] ~ N(0,1); and per-set arrays
    with a leading ring axis: x [K,S,H,R,P], B, C [K,S,H,R,N], dt, lam [K,S,H],
    theta [K,S,H,N/2] (plus *_raw storage arrays for x, B, C).  Step t uses
    set t mod K as the current token and set (t-1) mod K as the previous one.
    """
    rng = np.random.default_rng(seed)
    A = (-np.exp(rng.uniform(a_range[0], a_range[1], size=nheads))).astype(np.float32)
    h0 = rng.standard_normal((batch, nheads, N, P), dtype=np.float32)
    dt = _softplus(rng.standard_normal((ring, batch, nheads)) - 1.0).astype(np.float32)
    lam = _sigmoid(rng.standard_normal((ring, batch, nheads))).astype(np.float32)
    theta = rng.uniform(-np.pi, np.pi, size=(ring, batch, nheads, N // 2)).astype(np.float32)
    x32 = rng.standard_normal((ring, batch, nheads, R, P), dtype=np.float32)
    B32 = rng.standard_normal((ring, batch, nheads, R, N), dtype=np.float32)
    B32 *= np.float32(1.0 / np.sqrt(N))
    C32 = rng.standard_normal((ring, batch, nheads, R, N), dtype=np.float32)
    C32 *= np.float32(1.0 / np.sqrt(N))
    x, x_raw = _store(x32, dtype)
    Bv, B_raw = _store(B32, dtype)
    Cv, C_raw = _store(C32, dtype)
    return dict(A=A, h0=h0, x=x, B=Bv, C=Cv, x_raw=x_raw, B_raw=B_raw, C_raw=C_raw,
                dt=dt, lam=lam, theta=theta, dtype=dtype)


def decode_config_inputs(seed: Optional[int] = None, batch: Optional[int] = None,
                         ring: Optional[int] = None) -> Dict[str, np.ndarray]:
    cfg = WORKLOADS[4]
    return decode_inputs(batch=cfg.batch if batch is None else batch, nheads=cfg.nheads,
                         N=cfg.N, P=cfg.P, R=cfg.R, dtype=cfg.dtype,
                         ring=cfg.ring if ring is None else ring,
                         seed=4 if seed is None else seed)


def block_inputs(batch: int, seqlen: int, nheads: int, N: int, P: int, R: int, dtype: str,
                 seed: int) -> Dict[str, np.ndarray]:
    """Synthetic inputs and random weights of the block-side passes.

    Projection outputs before BCNorm: x ~ N(0,1) [B,T,H,P]; B, C ~ N(0,1)
    [B,T,H,R,N] (the raw projections, whose scale BCNorm removes).  Weights
    (float32, random -- no trained weights exist here): norm_B, norm_C ~
    U(0.5, 1.5) [H,N]; bias_B, bias_C ~ N(0, 0.1^2) [H,R,N]; up, down ~
    N(0, 1/R) [H,R,P].  Drawn in that order; x, B, C rounded to the storage
    dtype (returned as stored float32 values plus *_raw storage arrays).
    """
    rng = np.random.default_rng(seed)
    x32 = rng.standard_normal((batch, seqlen, nheads, P), dtype=np.float32)
    B32 = rng.standard_normal((batch, seqlen, nheads, R, N), dtype=np.float32)
    C32 = rng.standard_normal((batch, seqlen, nheads, R, N), dtype=np.float32)
    norm_B = rng.uniform(0.5, 1.5, size=(nheads, N)).astype(np.float32)
    norm_C = rng.uniform(0.5, 1.5, size=(nheads, N)).astype(np.float32)
    bias_B = (0.1 * rng.standard_normal((nheads, R, N))).astype(np.float32)
    bias_C = (0.1 * rng.standard_normal((nheads, R, N))).astype(np.float32)
    up = (rng.standard_normal((nheads, R, P)) / np.sqrt(R)).astype(np.float32)
    down = (rng.standard_normal((nheads, R, P)) / np.sqrt(R)).astype(np.float32)
    x, x_raw = _store(x32, dtype)
    Bv, B_raw = _store(B32, dtype)
    Cv, C_raw = _store(C32, dtype)
    return dict(x=x, B=Bv, C=Cv, x_raw=x_raw, B_raw=B_raw, C_raw=C_raw, norm_B=norm_B,
                norm_C=norm_C, bias_B=bias_B, bias_C=bias_C, up=up, down=down, dtype=dtype)
