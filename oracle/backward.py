"""fp64 oracle of the gradients of the SSM layer recurrence.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may use it;
it shares no code with the GPU library.

``forward`` writes the recurrence out in plain PyTorch CPU operations on
float64 tensors, step by step in time:

    h_t = alpha_t R_t ( h_{t-1} + (1 - lam_t) dt_t B_{t-1} x_{t-1}^T ) + lam_t dt_t B_t x_t^T
    y_t = C_t^T h_t

(Mamba-3 paper summary, Proposition 1; the complex transition as 2x2
rotations on row pairs (2k, 2k+1), explainer, "second improvement"; the
rank-R products of MIMO, paper summary, item 3), and ``gradients`` takes the
derivatives of  L = sum(y * dy) + sum(h_{T-1} * dh_final)  by PyTorch's
reverse-mode differentiation (a library primitive).  The forward is pinned to
the C oracle and the gradients to central finite differences of the C oracle
in ``tests/test_oracle_backward.py``.
"""
from __future__ import annotations

import numpy as np


def forward(x, dt, A, lam, theta, B, C):
    """float64 torch tensors: x [Bt,T,H,R,P]; dt, lam [Bt,T,H]; A [H];
    theta [Bt,T,H,N/2]; B, C [Bt,T,H,R,N].  Returns (y [Bt,T,H,R,P],
    h_final [Bt,H,N,P])."""
    import torch
    nb, nt, nh, nr, npd = x.shape
    nn = B.shape[-1]
    h = torch.zeros((nb, nh, nn, npd), dtype=torch.float64)
    prev = torch.zeros((nb, nh, nn, npd), dtype=torch.float64)  # B_{t-1} x_{t-1}^T
    ys = []
    for t in range(nt):
        d = dt[:, t]                                            # [Bt, H]
        alpha = torch.exp(d * A)
        psi = d[..., None] * theta[:, t]                        # [Bt, H, N/2]
        bx = torch.einsum("bhrn,bhrp->bhnp", B[:, t], x[:, t])
        u = h + ((1.0 - lam[:, t]) * d)[..., None, None] * prev
        cs, sn = torch.cos(psi)[..., None], torch.sin(psi)[..., None]
        u0, u1 = u[:, :, 0::2], u[:, :, 1::2]
        rot = torch.stack((cs * u0 - sn * u1, sn * u0 + cs * u1), dim=3).reshape(nb, nh, nn, npd)
        h = alpha[..., None, None] * rot + (lam[:, t] * d)[..., None, None] * bx
        prev = bx
        ys.append(torch.einsum("bhrn,bhnp->bhrp", C[:, t], h))
    return torch.stack(ys, dim=1), h


def gradients(x, dt, A, lam, theta, B, C, dy, dh_final=None):
    """Gradients of L = sum(y * dy) + sum(h_final * dh_final) with respect to
    x, dt, A, lam, theta, B, C (numpy float64 arrays, the inputs' shapes)."""
    import torch
    names = ("x", "dt", "A", "lam", "theta", "B", "C")
    ts = {k: torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True)
          for k, v in zip(names, (x, dt, A, lam, theta, B, C))}
    y, h = forward(*(ts[k] for k in names))
    loss = (y * torch.tensor(np.asarray(dy, dtype=np.float64))).sum()
    if dh_final is not None:
        loss = loss + (h * torch.tensor(np.asarray(dh_final, dtype=np.float64))).sum()
    loss.backward()
    return {k: ts[k].grad.numpy() for k in names}
