"""Pins of the gradient oracle (oracle/backward.py), CPU only.

The PyTorch forward is checked against the independent C oracle, and its
reverse-mode gradients against central finite differences of the C oracle
along random directions (central differences are second-order accurate:
at the step used their error is far below the tolerance), so neither the
forward written out here nor the differentiation is trusted on its own."""
import numpy as np
import pytest

import oracle
from oracle import backward


def problem(seed, nb=1, nt=9, nh=2, nr=2, npd=4, nn=6):
    rng = np.random.default_rng(seed)
    return dict(
        x=rng.standard_normal((nb, nt, nh, nr, npd)),
        dt=np.log1p(np.exp(rng.standard_normal((nb, nt, nh)) - 1.0)),
        A=-np.exp(rng.uniform(-2, 0, nh)),
        lam=1.0 / (1.0 + np.exp(-rng.standard_normal((nb, nt, nh)))),
        theta=rng.uniform(-np.pi, np.pi, (nb, nt, nh, nn // 2)),
        B=rng.standard_normal((nb, nt, nh, nr, nn)) / np.sqrt(nn),
        C=rng.standard_normal((nb, nt, nh, nr, nn)) / np.sqrt(nn))


def loss_c(p, dy, dhf):
    """L = sum(y * dy) + sum(h_final * dhf) through the C oracle (which reads
    its inputs as float32; the callers keep every input float32-exact)."""
    y, h = oracle.prefill(p["x"], p["dt"], p["A"], p["lam"], p["theta"], p["B"], p["C"])
    return float(np.sum(y * dy) + np.sum(h * dhf))


def test_forward_matches_c_oracle():
    import torch
    p = problem(1)
    y, h = backward.forward(*(torch.tensor(p[k]) for k in ("x", "dt", "A", "lam", "theta",
                                                           "B", "C")))
    # the C oracle reads its inputs as float32: give both the same values
    p32 = {k: v.astype(np.float32) for k, v in p.items()}
    y2, h2 = backward.forward(*(torch.tensor(p32[k].astype(np.float64))
                                for k in ("x", "dt", "A", "lam", "theta", "B", "C")))
    yc, hc = oracle.prefill(p32["x"], p32["dt"], p32["A"], p32["lam"], p32["theta"], p32["B"],
                            p32["C"])
    np.testing.assert_allclose(y2.numpy(), yc, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(h2.numpy(), hc, rtol=1e-12, atol=1e-13)
    assert y.shape == yc.shape


@pytest.mark.parametrize("seed", [2, 3])
def test_gradients_match_finite_differences(seed):
    """Directional derivatives along random directions: reverse-mode
    gradients against central differences of the C oracle's loss.  The C
    oracle rounds its inputs to float32, so the base point is float32-exact
    and the step is a multiple of each input's float32 spacing."""
    rng = np.random.default_rng(seed + 10)
    p = {k: v.astype(np.float32).astype(np.float64) for k, v in problem(seed).items()}
    dy = rng.standard_normal((1, 9, 2, 2, 4))
    dhf = rng.standard_normal((1, 2, 6, 4))
    g = backward.gradients(p["x"], p["dt"], p["A"], p["lam"], p["theta"], p["B"], p["C"], dy, dhf)
    for name in ("x", "dt", "A", "lam", "theta", "B", "C"):
        v = rng.standard_normal(p[name].shape)
        # a step of 2^-10 on float32-exact points keeps p +- eps*v float32-exact
        # only if v is a multiple of the spacing: round v to 2^-8 units
        v = np.round(v * 256.0) / 256.0
        eps = 2.0 ** -10
        plus, minus = dict(p), dict(p)
        plus[name] = p[name] + eps * v
        minus[name] = p[name] - eps * v
        fd = (loss_c(plus, dy, dhf) - loss_c(minus, dy, dhf)) / (2 * eps)
        ad = float(np.sum(g[name] * v))
        assert abs(fd - ad) <= 1e-4 * (abs(ad) + 1e-3), (name, fd, ad)


def test_lam_one_theta_zero_reduces_to_a_two_term_recurrence():
    """With lam = 1 and theta = 0 (the Mamba-2 rule) the gradient with
    respect to lam is still defined, and the x-gradient of a one-step
    sequence is dt * B^T C dy (y_0 = dt C^T B x_0^T for h_{-1} = 0)."""
    p = problem(4, nt=1)
    p["lam"][:] = 1.0
    p["theta"][:] = 0.0
    dy = np.random.default_rng(5).standard_normal((1, 1, 2, 2, 4))
    g = backward.gradients(p["x"], p["dt"], p["A"], p["lam"], p["theta"], p["B"], p["C"], dy)
    # y[r,p] = dt * sum_n C[n,r] sum_s B[n,s] x[s,p]  =>  dx[s,p] = dt sum_r (B^T C)[s,r] dy[r,p]
    for h in range(2):
        Bm, Cm = p["B"][0, 0, h], p["C"][0, 0, h]      # [R, N]
        ref = p["dt"][0, 0, h] * (Bm @ Cm.T) @ dy[0, 0, h]
        np.testing.assert_allclose(g["x"][0, 0, h], ref, rtol=1e-12)
