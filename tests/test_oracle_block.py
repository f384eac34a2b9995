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


# ---- hand-worked cases: each weight's axes and sign ---------------------------
# Rows of all ones (or all minus ones) have RMS exactly 1, so with eps = 0 the
# normalised row is +-w exactly and every expected value below is a short
# decimal written out by hand.


def test_bias_is_added_per_head_rank_channel_after_the_norm():
    """B rows of ones (RMS 1), norm weight 2: B~ = 2 + bias[h][r][n]; rows of
    minus ones give -2 + bias.  The bias differs per rank, per head and per
    channel, so dropping an axis, subtracting the bias or adding it before
    the normalisation all change the table."""
    nh, nr, nn = 2, 3, 4
    bias = np.array([[[0.0, 0.25, 0.5, 0.75], [1.0, 1.25, 1.5, 1.75], [2.0, 2.25, 2.5, 2.75]],
                     [[10.0, 10.25, 10.5, 10.75], [11.0, 11.25, 11.5, 11.75],
                      [12.0, 12.25, 12.5, 12.75]]])
    B = np.ones((1, 2, nh, nr, nn))
    B[0, 1] = -1.0                       # second token: rows of minus ones
    w = np.full((nh, nn), 2.0)
    x = np.zeros((1, 2, nh, 1))
    _, Bn, Cn = block.block_prepass(x, B, B, w, w, bias, bias, np.ones((nh, nr, 1)), 0.0)
    expect_pos = np.array([[[2.0, 2.25, 2.5, 2.75], [3.0, 3.25, 3.5, 3.75], [4.0, 4.25, 4.5, 4.75]],
                           [[12.0, 12.25, 12.5, 12.75], [13.0, 13.25, 13.5, 13.75],
                            [14.0, 14.25, 14.5, 14.75]]])
    expect_neg = np.array([[[-2.0, -1.75, -1.5, -1.25], [-1.0, -0.75, -0.5, -0.25],
                            [0.0, 0.25, 0.5, 0.75]],
                           [[8.0, 8.25, 8.5, 8.75], [9.0, 9.25, 9.5, 9.75],
                            [10.0, 10.25, 10.5, 10.75]]])
    np.testing.assert_array_equal(Bn[0, 0], expect_pos)
    np.testing.assert_array_equal(Bn[0, 1], expect_neg)
    np.testing.assert_array_equal(Cn, Bn)


def test_norm_weight_is_per_head_and_channel():
    """Rows of ones, zero bias: B~[h][r][n] = w[h][n] for every rank."""
    w = np.array([[0.5, 1.0, 1.5], [2.0, 4.0, 8.0]])
    B = np.ones((1, 1, 2, 2, 3))
    z = np.zeros((2, 2, 3))
    _, Bn, _ = block.block_prepass(np.zeros((1, 1, 2, 1)), B, B, w, w, z, z,
                                   np.ones((2, 2, 1)), 0.0)
    expect = np.array([[[0.5, 1.0, 1.5], [0.5, 1.0, 1.5]], [[2.0, 4.0, 8.0], [2.0, 4.0, 8.0]]])
    np.testing.assert_array_equal(Bn[0, 0], expect)


def test_rms_is_taken_per_row_over_the_state_channels():
    """Rank 0 holds [3, 4] and rank 1 [6, 8]: each row has its own RMS
    (sqrt 12.5 and sqrt 50), so both normalise to [3, 4] / sqrt(12.5) =
    [0.848528137423857, 1.131370849898476]; a norm over both ranks (mean
    square 31.25) or over the heads would not."""
    B = np.array([[[[[3.0, 4.0], [6.0, 8.0]], [[1.0, 1.0], [1.0, 1.0]]]]])  # [1,1,2,2,2]
    z = np.zeros((2, 2, 2))
    _, Bn, _ = block.block_prepass(np.zeros((1, 1, 2, 1)), B, B, np.ones((2, 2)), np.ones((2, 2)),
                                   z, z, np.ones((2, 2, 1)), 0.0)
    row = [0.848528137423857, 1.131370849898476]
    np.testing.assert_allclose(Bn[0, 0, 0, 0], row, rtol=1e-14)
    np.testing.assert_allclose(Bn[0, 0, 0, 1], row, rtol=1e-14)
    np.testing.assert_array_equal(Bn[0, 0, 1], [[1.0, 1.0], [1.0, 1.0]])


def test_up_projection_is_per_head_rank_channel():
    """x[h] = [1, 2] and [3, 4]; up[h][r] = [[2, 3], [5, 7]] and [[11, 13],
    [17, 19]]: X[h][r][p] = x[h][p] * up[h][r][p]."""
    x = np.array([[[[1.0, 2.0], [3.0, 4.0]]]])                       # [1,1,2,2]
    up = np.array([[[2.0, 3.0], [5.0, 7.0]], [[11.0, 13.0], [17.0, 19.0]]])
    B = np.ones((1, 1, 2, 2, 2))
    z = np.zeros((2, 2, 2))
    X, _, _ = block.block_prepass(x, B, B, np.ones((2, 2)), np.ones((2, 2)), z, z, up, 0.0)
    expect = np.array([[[2.0, 6.0], [5.0, 14.0]], [[33.0, 52.0], [51.0, 76.0]]])
    np.testing.assert_array_equal(X[0, 0], expect)


def test_down_projection_sums_the_ranks_per_head():
    """Head 0: y = [[1, 2], [3, 4], [5, 6]], down = [[1, 0.5], [2, 0.25],
    [-1, 1]] -> [1 + 6 - 5, 1 + 1 + 6] = [2, 8].  Head 1: same y, down =
    [[0, 1], [1, 0], [0.5, 0.5]] -> [0 + 3 + 2.5, 2 + 0 + 3] = [5.5, 5]."""
    yr = [[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]]
    y = np.array([[[yr, yr]]])                                        # [1,1,2,3,2]
    down = np.array([[[1.0, 0.5], [2.0, 0.25], [-1.0, 1.0]], [[0.0, 1.0], [1.0, 0.0], [0.5, 0.5]]])
    out = block.block_postpass(y, down)
    np.testing.assert_array_equal(out[0, 0], [[2.0, 8.0], [5.5, 5.0]])
