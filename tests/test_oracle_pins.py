"""Pins of the fp64 oracle against what the Mamba-3 pages and mathematics fix.

Each test checks the oracle (oracle/m3_oracle.c through oracle.prefill /
oracle.decode_step) against something other than itself: a special case that
reduces to the Mamba-2 rule, the parity-by-rotation construction, a closed
form steady state, the structured-mask form, the rotated-frame (RoPE)
recurrence, the order of accuracy against an exact ODE solution, MIMO
linearity, and split / invariance properties.  A plausible mistake in the
oracle (a dropped beta term, the beta term not rotated, a wrong sign of the
rotation, a transposed operand, an off-by-one in the previous input) fails at
least one of them.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import bruteforce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_problem(rng, nb, nt, nh, nr, npd, nn, a_range=(-2.0, 0.0)):
    """Small random problem (float32 values, like the real inputs)."""
    f = np.float32
    A = (-np.exp(rng.uniform(*a_range, size=nh))).astype(f)
    dt = np.logaddexp(0, rng.standard_normal((nb, nt, nh)) - 1).astype(f)
    lam = (1 / (1 + np.exp(-rng.standard_normal((nb, nt, nh))))).astype(f)
    theta = rng.uniform(-np.pi, np.pi, (nb, nt, nh, nn // 2)).astype(f)
    x = rng.standard_normal((nb, nt, nh, nr, npd)).astype(f)
    B = (rng.standard_normal((nb, nt, nh, nr, nn)) / np.sqrt(nn)).astype(f)
    C = (rng.standard_normal((nb, nt, nh, nr, nn)) / np.sqrt(nn)).astype(f)
    return dict(x=x, dt=dt, A=A, lam=lam, theta=theta, B=B, C=C)


def run(p, **kw):
    return oracle.prefill(p["x"], p["dt"], p["A"], p["lam"], p["theta"], p["B"], p["C"], **kw)


def rel(a, b):
    return np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300)


@pytest.fixture(scope="module", autouse=True)
def _built(oracle_lib):
    return oracle_lib


# ---------------------------------------------------------------------------
# P-1: lam = 1, theta = 0 is the Mamba-2 (exponential-Euler) rule
# (explainer: Mamba-1/2 discretisation h_t = e^{dt A} h + dt B x; paper summary,
#  Proposition 1: lam = 1 falls back to Euler; paper translation, Remark 5).
def test_p1_mamba2_reduction():
    rng = np.random.default_rng(11)
    p = rand_problem(rng, 2, 37, 3, 2, 5, 6)
    p["lam"][:] = 1.0
    p["theta"][:] = 0.0
    y, hf = run(p)
    x, dt, A, B, C = (p[k].astype(np.float64) for k in ("x", "dt", "A", "B", "C"))
    nb, nt, nh, nr, npd = x.shape
    nn = B.shape[-1]
    y_ref = np.zeros_like(y)
    h_ref = np.zeros_like(hf)
    for b in range(nb):
        for h in range(nh):
            st = np.zeros((nn, npd))
            for t in range(nt):
                st = np.exp(dt[b, t, h] * A[h]) * st + dt[b, t, h] * B[b, t, h].T @ x[b, t, h]
                y_ref[b, t, h] = C[b, t, h] @ st
            h_ref[b, h] = st
    assert rel(y, y_ref) < 1e-13
    assert rel(hf, h_ref) < 1e-13


# ---------------------------------------------------------------------------
# P-2: parity by rotation (paper translation section 3.2; explainer, second
# improvement).  Golden bit strings with their sign sequences.
def _golden_parity():
    rows = []
    with open(os.path.join(GOLDEN, "parity_construction.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            bits, signs = line.split()
            rows.append(([int(c) for c in bits], [1.0 if c == "+" else -1.0 for c in signs]))
    return rows


@pytest.mark.parametrize("lam_value", [1.0, 0.5, 0.0])
def test_p2_parity_rotation(lam_value):
    """With lam < 1 the previous-input term carries the seed into step 1; it
    must be rotated with the state, or the sign pattern breaks."""
    for bits, signs in _golden_parity():
        nt = len(bits)
        npd, nn = 3, 4
        p = dict(
            x=np.zeros((1, nt, 1, 1, npd), np.float32),
            dt=np.ones((1, nt, 1), np.float32),
            A=np.zeros(1, np.float32),
            lam=np.full((1, nt, 1), lam_value, np.float32),
            theta=np.zeros((1, nt, 1, nn // 2), np.float32),
            B=np.zeros((1, nt, 1, 1, nn), np.float32),
            C=np.zeros((1, nt, 1, 1, nn), np.float32),
        )
        p["theta"][0, :, 0, :] = (np.pi * np.array(bits, np.float64))[:, None].astype(np.float32)
        x0 = np.array([0.5, -1.25, 2.0], np.float32)
        b0 = np.array([1.0, 0.25, -0.5, 0.75], np.float32)
        p["x"][0, 0, 0, 0] = x0
        p["B"][0, 0, 0, 0] = b0
        p["B"][0, 1:, 0, 0] = 3.0          # B of later steps must not matter (x = 0 there)
        p["C"][0, :, 0, 0] = np.array([1.0, 0.0, 0.0, 1.0], np.float32)
        # pi in float32 is not exactly pi: compare with the sign pattern at 1e-6
        seed = np.outer(b0, x0).astype(np.float64)
        nb_steps = len(signs)
        for t in range(nb_steps):
            pp = {k: (v[:, :t + 1] if v.ndim >= 2 and k != "A" else v) for k, v in p.items()}
            y, hf = run(pp)
            # step 0 holds lam * seed (lam = 0 -> the seed enters at step 1)
            scale = lam_value if t == 0 else 1.0
            np.testing.assert_allclose(hf[0, 0], signs[t] * scale * seed, atol=1e-6)
            np.testing.assert_allclose(y[0, t, 0, 0], signs[t] * scale * (seed[0] + seed[3]),
                                       atol=1e-6)


# ---------------------------------------------------------------------------
# P-3: closed-form steady state of constant inputs (fixed point of the
# complex recurrence: z = ((1-lam) dt a_c + lam dt) v / (1 - a_c)).
@pytest.mark.parametrize("theta_zero", [True, False])
def test_p3_steady_state(theta_zero):
    rng = np.random.default_rng(3)
    nn, npd, nr, nt = 6, 4, 2, 400
    dt, lam, A = 0.7, 0.35, -0.9
    theta = np.zeros(nn // 2) if theta_zero else rng.uniform(-np.pi, np.pi, nn // 2)
    x = rng.standard_normal((nr, npd))
    B = rng.standard_normal((nr, nn)) / 3
    C = rng.standard_normal((nr, nn)) / 3
    f = np.float32
    p = dict(
        x=np.broadcast_to(x.astype(f), (1, nt, 1, nr, npd)).copy(),
        dt=np.full((1, nt, 1), dt, f), A=np.array([A], f),
        lam=np.full((1, nt, 1), lam, f),
        theta=np.broadcast_to(theta.astype(f), (1, nt, 1, nn // 2)).copy(),
        B=np.broadcast_to(B.astype(f), (1, nt, 1, nr, nn)).copy(),
        C=np.broadcast_to(C.astype(f), (1, nt, 1, nr, nn)).copy(),
    )
    assert np.exp(f(dt) * f(A) * nt) < 1e-15
    y, hf = run(p)
    d, la, a = float(f(dt)), float(f(lam)), float(f(A))
    th = theta.astype(f).astype(np.float64)
    xs, Bs, Cs = (v.astype(f).astype(np.float64) for v in (x, B, C))
    ac = np.exp(d * (a + 1j * th))                               # [K]
    bc = Bs[:, 0::2] + 1j * Bs[:, 1::2]                          # [R, K]
    v = np.einsum("rk,rp->kp", bc, xs)                           # [K, P]
    z = (((1 - la) * d * ac + la * d) / (1 - ac))[:, None] * v
    h_star = np.empty((nn, npd))
    h_star[0::2], h_star[1::2] = z.real, z.imag
    np.testing.assert_allclose(hf[0, 0], h_star, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y[0, -1, 0], Cs @ h_star, rtol=1e-12, atol=1e-12)
    if theta_zero:  # real case: h = (beta + gamma) B x^T / (1 - alpha)
        al = np.exp(d * a)
        np.testing.assert_allclose(hf[0, 0], ((1 - la) * d * al + la * d) / (1 - al) * Bs.T @ xs,
                                   rtol=1e-12)


# ---------------------------------------------------------------------------
# P-4: brute-force structured-mask form, T <= 8 (and a few longer).
@pytest.mark.parametrize("shape", [
    (1, 1, 1, 1, 1, 2),     # nb, nt, nh, nr, P, N
    (1, 8, 1, 1, 3, 4),
    (2, 7, 2, 2, 5, 6),
    (1, 8, 3, 4, 4, 8),
    (1, 24, 2, 3, 3, 10),
])
def test_p4_bruteforce_masked_form(shape):
    nb, nt, nh, nr, npd, nn = shape
    rng = np.random.default_rng(sum(shape))
    p = rand_problem(rng, nb, nt, nh, nr, npd, nn)
    y, hf = run(p)
    y_bf, h_bf = bruteforce.masked_form(p["x"], p["dt"], p["A"], p["lam"], p["theta"], p["B"], p["C"])
    assert rel(y, y_bf) < 1e-12
    assert rel(hf, h_bf) < 1e-12


# ---------------------------------------------------------------------------
# P-5: rotated-frame (data-dependent RoPE, Proposition 3 with the trapezoid
# terms) recurrence equals the complex recurrence, for y and the final state.
def rotated_frame(p):
    x, dt, A, lam, theta, B, C = (np.asarray(p[k], np.float64)
                                  for k in ("x", "dt", "A", "lam", "theta", "B", "C"))
    nb, nt, nh, nr, npd = x.shape
    nn = B.shape[-1]
    y = np.zeros((nb, nt, nh, nr, npd))
    hf = np.zeros((nb, nh, nn, npd))
    for b in range(nb):
        for h in range(nh):
            phi = np.cumsum(dt[b, :, h, None] * theta[b, :, h], axis=0)   # [T, K]
            c, s = np.cos(phi), np.sin(phi)

            def rot_t(v):  # R(phi)^T applied to pairs of v [T, R, N]
                out = np.empty_like(v)
                v0, v1 = v[..., 0::2], v[..., 1::2]
                out[..., 0::2] = c[:, None] * v0 + s[:, None] * v1
                out[..., 1::2] = -s[:, None] * v0 + c[:, None] * v1
                return out

            Bt, Ct = rot_t(B[b, :, h]), rot_t(C[b, :, h])
            st = np.zeros((nn, npd))
            prev = np.zeros((nn, npd))
            for t in range(nt):
                al = np.exp(dt[b, t, h] * A[h])
                cur = Bt[t].T @ x[b, t, h]
                st = al * st + (1 - lam[b, t, h]) * dt[b, t, h] * al * prev + lam[b, t, h] * dt[b, t, h] * cur
                prev = cur
                y[b, t, h] = Ct[t] @ st
            out = np.empty_like(st)
            c1, s1 = c[-1][:, None], s[-1][:, None]
            out[0::2] = c1 * st[0::2] - s1 * st[1::2]
            out[1::2] = s1 * st[0::2] + c1 * st[1::2]
            hf[b, h] = out
    return y, hf


def test_p5_rope_trick_equivalence():
    rng = np.random.default_rng(5)
    p = rand_problem(rng, 2, 50, 2, 2, 4, 8)
    y, hf = run(p)
    y_r, h_r = rotated_frame(p)
    assert rel(y, y_r) < 1e-12
    assert rel(hf, h_r) < 1e-12


def test_p5_first_angle_cancels():
    """The angle of step 0 acts on nothing (zero state, no previous input)."""
    rng = np.random.default_rng(6)
    p = rand_problem(rng, 1, 20, 2, 1, 3, 4)
    y1, h1 = run(p)
    p["theta"][:, 0] = rng.uniform(-np.pi, np.pi, p["theta"][:, 0].shape).astype(np.float32)
    y2, h2 = run(p)
    assert rel(y2, y1) < 1e-14 and rel(h2, h1) < 1e-14
    p["theta"][:, 1] += np.float32(0.5)
    y3, _ = run(p)
    assert rel(y3, y1) > 1e-3


# ---------------------------------------------------------------------------
# P-6: order of accuracy on a scalar complex ODE with an exact solution
# (paper summary, item 1: trapezoid is second order, Euler first order;
# explainer: O(dt^3) local error for lam near 1/2).
def _ode_error(lam_value, n_steps, beta_rotated=True):
    a, w, t_end = -0.5, 3.0, 2.0
    bc = 1.0 + 0.5j
    mu = a + 1j * w
    d = t_end / n_steps
    tk = np.arange(n_steps + 1) * d
    u = np.sin(tk)
    # exact: z(t) = b [ e^{mu t} - (mu sin t + cos t) ] / (1 + mu^2), z(0) = 0
    z_exact = bc * (np.exp(mu * t_end) - (mu * np.sin(t_end) + np.cos(t_end))) / (1 + mu ** 2)
    if beta_rotated:
        nt = n_steps + 1
        y, hf = oracle.prefill(
            u.reshape(1, nt, 1, 1, 1), np.full((1, nt, 1), d), np.array([a]),
            np.full((1, nt, 1), lam_value), np.full((1, nt, 1, 1), w),
            np.broadcast_to(np.array([bc.real, bc.imag]), (1, nt, 1, 1, 2)),
            np.broadcast_to(np.array([1.0, 0.0]), (1, nt, 1, 1, 2)))
        z = hf[0, 0, 0, 0] + 1j * hf[0, 0, 1, 0]
    else:  # the misreading: beta = (1-lam) dt e^{dt A} without the rotation
        z = 0.0
        for k in range(1, n_steps + 1):
            z = np.exp(mu * d) * z + (1 - lam_value) * d * np.exp(a * d) * bc * u[k - 1] + lam_value * d * bc * u[k]
    return abs(z - z_exact)


def test_p6_order_of_accuracy():
    # float32 inputs are accepted as given: use step counts whose dt is exact
    ratios_trap = [_ode_error(0.5, n) / _ode_error(0.5, 2 * n) for n in (64, 128, 256)]
    ratios_euler = [_ode_error(1.0, n) / _ode_error(1.0, 2 * n) for n in (64, 128, 256)]
    ratios_wrong = [_ode_error(0.5, n, False) / _ode_error(0.5, 2 * n, False) for n in (64, 128, 256)]
    assert all(3.8 < r < 4.2 for r in ratios_trap), ratios_trap
    assert all(1.8 < r < 2.2 for r in ratios_euler), ratios_euler
    assert all(r < 2.3 for r in ratios_wrong), ratios_wrong


# ---------------------------------------------------------------------------
# P-7: MIMO is the rank-R sum of SISO updates (paper summary, item 3;
# explainer, third improvement).
def test_p7_mimo_linearity():
    rng = np.random.default_rng(7)
    nr = 3
    p = rand_problem(rng, 1, 30, 2, nr, 4, 6)
    y, hf = run(p)
    y_sum = np.zeros_like(y)
    h_sum = np.zeros_like(hf)
    for r_in in range(nr):
        for r_out in range(nr):
            q = dict(p)
            q["x"] = p["x"][:, :, :, r_in:r_in + 1]
            q["B"] = p["B"][:, :, :, r_in:r_in + 1]
            q["C"] = p["C"][:, :, :, r_out:r_out + 1]
            ys, hs = run(q)
            y_sum[:, :, :, r_out] += ys[:, :, :, 0]
            if r_out == 0:
                h_sum += hs
    assert rel(y, y_sum) < 1e-12
    assert rel(hf, h_sum) < 1e-12
    # R = 1 MIMO is SISO: superposition in x
    q = dict(p)
    q["x"], q["B"], q["C"] = p["x"][:, :, :, :1], p["B"][:, :, :, :1], p["C"][:, :, :, :1]
    q2 = dict(q)
    q2["x"] = 2.0 * q["x"]
    ya, ha = run(q)
    yb, hb = run(q2)
    assert rel(yb, 2 * ya) < 1e-14 and rel(hb, 2 * ha) < 1e-14


# ---------------------------------------------------------------------------
# Split invariance: a prefix run then a continuation from (h, previous token)
# equals one run over the whole sequence; the decode step reproduces prefill.
def test_continuation_split():
    rng = np.random.default_rng(8)
    p = rand_problem(rng, 2, 41, 2, 2, 3, 6)
    y, hf = run(p)
    cut = 17
    a = {k: (v[:, :cut] if k != "A" else v) for k, v in p.items()}
    b = {k: (v[:, cut:] if k != "A" else v) for k, v in p.items()}
    ya, ha = run(a)
    yb, hb = run(b, h0=ha, x_halo=p["x"][:, cut - 1], B_halo=p["B"][:, cut - 1])
    assert rel(np.concatenate([ya, yb], axis=1), y) < 1e-13
    assert rel(hb, hf) < 1e-13
    # without the halo the beta term of the first continued step is lost
    yc, _ = run(b, h0=ha)
    assert rel(np.concatenate([ya, yc], axis=1), y) > 1e-4


def test_decode_matches_prefill_and_units():
    rng = np.random.default_rng(9)
    nb, nt, nh, nr, npd, nn = 3, 12, 2, 2, 4, 6
    p = rand_problem(rng, nb, nt, nh, nr, npd, nn)
    y, hf = run(p)
    h = np.zeros((nb, nh, nn, npd))
    xp = np.zeros((nb, nh, nr, npd), np.float32)
    bp = np.zeros((nb, nh, nr, nn), np.float32)
    for t in range(nt):
        yt, h = oracle.decode_step(h, p["x"][:, t], xp, p["B"][:, t], bp, p["C"][:, t],
                                   p["dt"][:, t], p["A"], p["lam"][:, t], p["theta"][:, t])
        assert rel(yt, y[:, t]) < 1e-13
        xp, bp = p["x"][:, t], p["B"][:, t]
    assert rel(h, hf) < 1e-13
    # a unit subset computes exactly the same numbers for those units
    yu, hu = run(p, units=[4, 1])
    for u in (4, 1):
        b_, h_ = divmod(u, nh)
        np.testing.assert_array_equal(yu[b_, :, h_], y[b_, :, h_])
        np.testing.assert_array_equal(hu[b_, h_], hf[b_, h_])
    assert np.isnan(yu[0, :, 0]).all()


def test_threads_do_not_change_results():
    rng = np.random.default_rng(10)
    p = rand_problem(rng, 2, 33, 3, 1, 4, 8)
    y1, h1 = run(p, nthreads=1)
    y4, h4 = run(p, nthreads=4)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(h1, h4)
