"""Second, independent fp64 formulation of the Mamba-3 recurrence: the
parallel structured-mask ("SSD") form, for short sequences only.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

It does not run the recurrence.  It builds, in plain NumPy:

* the cumulative rotation P_t = prod_{i<=t} R_i^T (explicit 2x2 matrix
  products per pair), and the rotated inputs B~_t = P_t B_t, C~_t = P_t C_t
  -- the data-dependent RoPE of Proposition 3 (Mamba-3 paper summary,
  aipaper.cc, "Mathematical formulas", item 2; Mamba-3 paper translation,
  sz-guanghua.com.cn, section 3.2.1);
* the T x T decay matrix L[t,s] = prod_{s<i<=t} alpha_i (lower triangular,
  semiseparable) and the 2-band matrix D with gamma_t on the diagonal and
  beta_t on the sub-diagonal; the mask is the product L @ D (paper
  translation, section 3.1, equation 7 and Remark 5; explainer, yunpan.plus,
  "training and inference both benefit");
* y_t[r] = sum_u (L D)[t,u] * sum_r' (C~_t[r] . B~_u[r']) x_u[r'], and the
  final state h_{T-1} = P_{T-1}^T * sum_u (L D)[T-1,u] sum_r' B~_u[r'] x_u[r']^T.

Rotation convention: R(phi) = [[cos phi, -sin phi], [sin phi, cos phi]]
acting on the pair (2k, 2k+1), phi = dt_t * theta_t[k].
"""
from __future__ import annotations

import numpy as np


def _rot(phi):
    """2x2 rotation matrices for an array of angles -> [..., 2, 2]."""
    c, s = np.cos(phi), np.sin(phi)
    out = np.empty(phi.shape + (2, 2))
    out[..., 0, 0] = c
    out[..., 0, 1] = -s
    out[..., 1, 0] = s
    out[..., 1, 1] = c
    return out


def masked_form(x, dt, A, lam, theta, B, C):
    """Structured-mask evaluation for one batch of short sequences.

    Shapes as the oracle: x [Bt,T,H,R,P]; B, C [Bt,T,H,R,N]; dt, lam
    [Bt,T,H]; theta [Bt,T,H,N/2]; A [H].  Returns (y, h_final) in float64.
    Cost is O(T^2) per unit: meant for T <= ~64.
    """
    x, dt, A, lam, theta, B, C = (np.asarray(a, dtype=np.float64)
                                  for a in (x, dt, A, lam, theta, B, C))
    nb, nt, nh, nr, npd = x.shape
    nn = B.shape[-1]
    npair = nn // 2
    y = np.zeros((nb, nt, nh, nr, npd))
    hf = np.zeros((nb, nh, nn, npd))
    for b in range(nb):
        for h in range(nh):
            d = dt[b, :, h]
            la = lam[b, :, h]
            alpha = np.exp(d * A[h])
            beta = (1.0 - la) * d * alpha
            gamma = la * d
            # cumulative rotations P_t = R_t^T ... R_0^T (2x2 per pair)
            Rt = _rot(d[:, None] * theta[b, :, h, :])            # [T, npair, 2, 2]
            Pc = np.empty_like(Rt)
            acc = np.broadcast_to(np.eye(2), (npair, 2, 2)).copy()
            for t in range(nt):
                acc = np.einsum("kij,kjl->kil", np.swapaxes(Rt[t], -1, -2), acc)
                Pc[t] = acc
            Bp = B[b, :, h].reshape(nt, nr, npair, 2)
            Cp = C[b, :, h].reshape(nt, nr, npair, 2)
            Bt = np.einsum("tkij,trkj->trki", Pc, Bp).reshape(nt, nr, nn)
            Ct = np.einsum("tkij,trkj->trki", Pc, Cp).reshape(nt, nr, nn)
            # decay matrix L and 2-band matrix D
            L = np.zeros((nt, nt))
            for t in range(nt):
                for s in range(t + 1):
                    L[t, s] = np.prod(alpha[s + 1:t + 1])
            D = np.diag(gamma)
            for t in range(1, nt):
                D[t, t - 1] = beta[t]
            M = L @ D
            xs = x[b, :, h]                                        # [T, R, P]
            scores = np.einsum("trn,usn->trus", Ct, Bt)            # [T,R,T,R]
            y[b, :, h] = np.einsum("tu,trus,usp->trp", M, scores, xs)
            hrot = np.einsum("u,usn,usp->np", M[nt - 1], Bt, xs)   # rotated frame
            hr = hrot.reshape(npair, 2, npd)
            hf[b, h] = np.einsum("kji,kjp->kip", Pc[nt - 1], hr).reshape(nn, npd)
    return y, hf
