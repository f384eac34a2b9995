"""Pins of the block-side oracle (oracle/block.py) against closed forms,
invariants and an explicit-loop computation on tiny inputs (CPU only).

Sources: Mamba-3 paper translation, section 3.4 (BCNorm as an RMS
normalisation after the B, C projections; a head-specific channel-wise bias
after it) and section 3.3 (MIMO projections P -> P x R -> P with additive
parameter growth)."""
import math

import numpy as np

from oracle import block


def test_constant_row_normalises_to_its_sign():
    """A row whose N entries all equal c has RMS |c|: with eps = 0 it
    normalises to sign(c) * w exactly."""
    w = np.linspace(0.5, 2.0, 8)
    for c in (3.0, -0.25, 1e-3):
        out = block.rms_norm(np.full(8, c), w, 0.0)
        np.testing.assert_allclose(out, np.sign(c) * w, rtol=1e-15, atol=0)


def test_hand_worked_row():
    """[3, 4]: mean square 12.5, so the row becomes [3, 4] / sqrt(12.5)."""
    out = block.rms_norm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.0)
    s = math.sqrt(12.5)
    np.testing.assert_allclose(out, [3.0 / s, 8.0 / s], rtol=1e-15)
    # eps enters under the root: mean square 12.5 + 0.5 = 13
    out = block.rms_norm(np.array([3.0, 4.0]), np.ones(2), 0.5)
    np.testing.assert_allclose(out, [3.0 / math.sqrt(13.0), 4.0 / math.sqrt(13.0)], rtol=1e-15)


def test_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((5, 64))
    a = block.rms_norm(v, np.ones(64), 0.0)
    b = block.rms_norm(7.5 * v, np.ones(64), 0.0)
    np.testing.assert_allclose(a, b, rtol=1e-13)
    np.testing.assert_allclose(np.mean(a * a, axis=-1), 1.0, rtol=1e-13)


def _loops_prepass(x, B, C, nB, nC, bB, bC, up, eps):
    nb, nt, nh, nr, nn = B.shape
    npd = x.shape[-1]
    X = np.zeros((nb, nt, nh, nr, npd))
    Bo = np.zeros(B.shape)
    Co = np.zeros(C.shape)
    for b in range(nb):
        for t in range(nt):
            for h in range(nh):
                for r in range(nr):
                    for src, w, bias, dst in ((B, nB, bB, Bo), (C, nC, bC, Co)):
                        ss = 0.0
                        for n in range(nn):
                            ss += float(src[b, t, h, r, n]) ** 2
                        scale = 1.0 / math.sqrt(ss / nn + eps)
                        for n in range(nn):
                            dst[b, t, h, r, n] = src[b, t, h, r, n] * scale * w[h, n] + bias[h, r, n]
                    for p in range(npd):
                        X[b, t, h, r, p] = x[b, t, h, p] * up[h, r, p]
    return X, Bo, Co


def test_prepass_and_postpass_against_loops():
    rng = np.random.default_rng(5)
    nb, nt, nh, nr, nn, npd = 2, 3, 2, 3, 6, 4
    x = rng.standard_normal((nb, nt, nh, npd))
    B = rng.standard_normal((nb, nt, nh, nr, nn))
    C = rng.standard_normal((nb, nt, nh, nr, nn))
    nB, nC = rng.uniform(0.5, 1.5, (nh, nn)), rng.uniform(0.5, 1.5, (nh, nn))
    bB, bC = rng.standard_normal((nh, nr, nn)), rng.standard_normal((nh, nr, nn))
    up = rng.standard_normal((nh, nr, npd))
    got = block.block_prepass(x, B, C, nB, nC, bB, bC, up, 1e-5)
    ref = _loops_prepass(x, B, C, nB, nC, bB, bC, up, 1e-5)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-13, atol=1e-14)
    y = rng.standard_normal((nb, nt, nh, nr, npd))
    down = rng.standard_normal((nh, nr, npd))
    out = block.block_postpass(y, down)
    for b in range(nb):
        for t in range(nt):
            for h in range(nh):
                for p in range(npd):
                    s = sum(y[b, t, h, r, p] * down[h, r, p] for r in range(nr))
                    assert abs(out[b, t, h, p] - s) <= 1e-13 * (1 + abs(s))


def test_single_rank_unit_projections_are_identity():
    """R = 1 with unit projections: X = x and the post-pass returns y."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 4, 2, 8))
    B = rng.standard_normal((1, 4, 2, 1, 16))
    X, _, _ = block.block_prepass(x, B, B, np.ones((2, 16)), np.ones((2, 16)),
                                  np.zeros((2, 1, 16)), np.zeros((2, 1, 16)),
                                  np.ones((2, 1, 8)), 1e-6)
    np.testing.assert_array_equal(X[:, :, :, 0], x)
    y = rng.standard_normal((1, 4, 2, 1, 8))
    np.testing.assert_array_equal(block.block_postpass(y, np.ones((2, 1, 8))), y[:, :, :, 0])
