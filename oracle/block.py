"""fp64 oracle of the block-side steps on either side of the SSM.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may use it;
it shares no code with the GPU library.

What the pages fix (Mamba-3 paper translation, section 3.4 "Mamba-3
architecture"; paper summary, "Steps & Procedures" items 3 and 5):

* BCNorm: an RMS normalisation added after the B and C projections, in the
  manner of QK normalisation.  Read here as RMSNorm over the N state
  channels of each (token, head, rank) row, with a learned per-head scale:
  v / sqrt(mean(v^2) + eps) * w.
* B, C bias: a learnable, head-specific, channel-wise bias added after
  BCNorm.  Read here as one bias per (head, rank, channel).
* MIMO projections (paper translation, section 3.3): the input is projected
  from P to P x R and the output back from P x R to P, with the parameter
  growth made additive rather than multiplicative (the details sit in an
  appendix the pages do not include).  Read here as per-head, per-rank
  channel-wise scalings: X_r = x * U_r and y = sum_r D_r * Y_r, which add
  2 R P parameters per head.

Each function is pinned in ``tests/test_oracle_block.py``.
"""
from __future__ import annotations

import numpy as np


def rms_norm(v, weight, eps):
    """RMS normalisation over the last axis, then the per-channel scale."""
    v = np.asarray(v, dtype=np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * np.asarray(weight, dtype=np.float64)


def block_prepass(x, B, C, norm_B, norm_C, bias_B, bias_C, up, eps):
    """x [Bt,T,H,P]; B, C [Bt,T,H,R,N]; norm_B, norm_C [H,N];
    bias_B, bias_C [H,R,N]; up [H,R,P].  Returns (X [Bt,T,H,R,P],
    B~ [Bt,T,H,R,N], C~ [Bt,T,H,R,N]) in float64: the SSM's inputs."""
    x = np.asarray(x, dtype=np.float64)
    nB = np.asarray(norm_B, dtype=np.float64)[None, None, :, None, :]
    nC = np.asarray(norm_C, dtype=np.float64)[None, None, :, None, :]
    Bn = rms_norm(B, nB, eps) + np.asarray(bias_B, dtype=np.float64)[None, None]
    Cn = rms_norm(C, nC, eps) + np.asarray(bias_C, dtype=np.float64)[None, None]
    X = x[:, :, :, None, :] * np.asarray(up, dtype=np.float64)[None, None]
    return X, Bn, Cn


def block_postpass(y, down):
    """y [Bt,T,H,R,P]; down [H,R,P] -> [Bt,T,H,P] float64."""
    y = np.asarray(y, dtype=np.float64)
    return np.sum(y * np.asarray(down, dtype=np.float64)[None, None], axis=3)
