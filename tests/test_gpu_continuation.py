"""GPU parity of prefill continuation (m3_prefill_from_state) against the fp64
oracle, through the C ABI.

A sequence processed in pieces -- each piece starting from the previous
piece's final state and last token -- must give the result of one pass over
the whole sequence (the chunked form chains chunks by the recurrence on the
state, so a piece boundary is one more chunk boundary).  Arbitrary initial
states and previous tokens are checked against the oracle's own continuation
(pinned on the CPU by the split test).  Tolerance as for prefill: rel-L2
<= 1e-4 (fp32 inputs), <= 2e-2 (bf16 inputs), for y and the final state."""
import numpy as np
import pytest

from state_space_sequence_exp_amd import inputs as I

from gpu_util import (TOL, from_gpu, log, oracle_threads, rel_l2, to_gpu_f32, to_gpu_storage,
                      upload_prefill)

pytestmark = pytest.mark.gpu


def run_pieces(g, cuts, chunk):
    """Prefill over [0, T) split at `cuts`, each piece continuing the last."""
    import state_space_sequence_exp_amd as m3
    T = g["x"].shape[1]
    bounds = [0] + list(cuts) + [T]
    ys, h, xp, bp = [], None, None, None
    for t0, t1 in zip(bounds[:-1], bounds[1:]):
        sl = {k: (g[k][:, t0:t1].contiguous() if k != "A" else g[k]) for k in g}
        y, h = m3.prefill(sl["x"], sl["dt"], sl["A"], sl["lam"], sl["theta"], sl["B"], sl["C"],
                          chunk, h0=h, x_prev=xp, B_prev=bp)
        ys.append(y)
        if t1 > t0:
            xp = g["x"][:, t1 - 1].contiguous()
            bp = g["B"][:, t1 - 1].contiguous()
    import torch
    return torch.cat(ys, dim=1), h


def oracle_full(inp, **kw):
    import oracle
    return oracle.prefill(inp["x"], inp["dt"], inp["A"], inp["lam"], inp["theta"], inp["B"],
                          inp["C"], nthreads=oracle_threads(), **kw)


# (dtype, batch, T, heads, N, P, R, chunk, cuts)
SPLITS = [
    ("f32", 1, 200, 2, 32, 32, 1, 32, (96,)),          # cut on a chunk boundary
    ("f32", 2, 150, 1, 16, 64, 2, 16, (1, 77)),        # a one-token piece, a ragged cut
    ("bf16", 2, 300, 2, 64, 64, 1, 64, (100, 101, 230)),
    ("bf16", 1, 260, 2, 128, 64, 1, 64, (130,)),
    ("bf16", 1, 180, 2, 64, 64, 4, 64, (64, 179)),     # MIMO, a one-token last piece
    ("bf16", 1, 1000, 1, 64, 64, 1, 32, (333, 667)),   # many segments per piece
    ("bf16", 4, 1500, 16, 64, 64, 1, 64, (700,)),      # single pass, segments of 3 and 4 chunks
    ("bf16", 4, 4096, 16, 64, 64, 1, 64, (2048,)),     # single pass, 8-chunk segments, no direct one
]


@pytest.mark.parametrize("case", SPLITS, ids=lambda c: "%s-t%d-n%d-p%d-r%d-l%d-cuts%s" % (
    c[0], c[2], c[4], c[5], c[6], c[7], "_".join(map(str, c[8]))))
def test_pieces_equal_one_pass(case):
    dtype, nb, T, nh, N, P, R, chunk, cuts = case
    log("continuation split %s" % (case,))
    inp = I.prefill_inputs(nb, T, nh, N, P, R, dtype, seed=70 + T)
    g = upload_prefill(inp)
    y, h = run_pieces(g, cuts, chunk)
    y_ref, h_ref = oracle_full(inp)
    ey, eh = rel_l2(from_gpu(y), y_ref), rel_l2(from_gpu(h), h_ref)
    log("  rel-L2 y %.2e  h %.2e" % (ey, eh))
    assert ey <= TOL[dtype] and eh <= TOL[dtype]


@pytest.mark.parametrize("dtype,with_h0,with_halo", [
    ("f32", True, True), ("f32", True, False), ("f32", False, True),
    ("bf16", True, True), ("bf16", True, False), ("bf16", False, True)])
def test_given_state_and_previous_token(dtype, with_h0, with_halo):
    """Arbitrary h0 and previous token (token 0 of a longer draw) against the
    oracle started from the same state and halo."""
    import state_space_sequence_exp_amd as m3
    nb, T, nh, N, P, R, chunk = 2, 140, 2, 64, 32, 2, 32
    full = I.prefill_inputs(nb, T + 1, nh, N, P, R, dtype, seed=81)
    rest = {k: (v[:, 1:] if isinstance(v, np.ndarray) and v.ndim >= 3 else v)
            for k, v in full.items()}
    g = upload_prefill(rest)
    h0 = np.random.default_rng(82).standard_normal((nb, nh, N, P)).astype(np.float32)
    kw, okw = {}, {}
    if with_h0:
        kw["h0"] = to_gpu_f32(h0)
        okw["h0"] = h0.astype(np.float64)
    if with_halo:
        kw["x_prev"] = to_gpu_storage(np.ascontiguousarray(full["x_raw"][:, 0]), dtype)
        kw["B_prev"] = to_gpu_storage(np.ascontiguousarray(full["B_raw"][:, 0]), dtype)
        okw["x_halo"] = full["x"][:, 0]
        okw["B_halo"] = full["B"][:, 0]
    y, h = m3.prefill(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"], chunk, **kw)
    y_ref, h_ref = oracle_full(rest, **okw)
    ey, eh = rel_l2(from_gpu(y), y_ref), rel_l2(from_gpu(h), h_ref)
    log("from-state %s h0=%s halo=%s: rel-L2 y %.2e  h %.2e" % (dtype, with_h0, with_halo, ey, eh))
    assert ey <= TOL[dtype] and eh <= TOL[dtype]
    # the effect of the given state and token on y, y(state) - y(zero state),
    # matches the oracle's: the halo alone moves y by only a few percent, so
    # this is what shows it was used (ignoring it gives an error of 1).  The
    # bound allows each output's bf16 rounding against a small difference.
    y0, _ = m3.prefill(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"], chunk)
    y0_ref, _ = oracle_full(rest)
    ed = rel_l2(from_gpu(y) - from_gpu(y0), y_ref - y0_ref)
    log("  effect of the state: rel-L2 %.2e" % ed)
    assert ed <= (1e-2 if dtype == "f32" else 0.2)


def test_in_place_state_update():
    """h_final may be h0 itself; the result equals the out-of-place one bit for bit."""
    import state_space_sequence_exp_amd as m3
    inp = I.prefill_inputs(2, 500, 2, 64, 64, 1, "bf16", seed=83)
    g = upload_prefill(inp)
    h0 = to_gpu_f32(np.random.default_rng(84).standard_normal((2, 2, 64, 64)))
    args = (g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"], 32)
    y1, h1 = m3.prefill(*args, h0=h0)
    h_in_place = h0.clone()
    y2, h2 = m3.prefill(*args, h0=h_in_place, h_final=h_in_place)
    assert h2.data_ptr() == h_in_place.data_ptr()
    assert np.array_equal(from_gpu(y1), from_gpu(y2))
    assert np.array_equal(from_gpu(h1), from_gpu(h2))


def test_empty_piece_passes_the_state_through():
    import torch
    import state_space_sequence_exp_amd as m3
    inp = I.prefill_inputs(2, 0, 3, 32, 16, 1, "bf16", seed=85)
    g = upload_prefill(inp)
    h0 = torch.randn(2, 3, 32, 16, device="cuda:0")
    xp = torch.randn(2, 3, 16, device="cuda:0").to(torch.bfloat16)
    bp = torch.randn(2, 3, 32, device="cuda:0").to(torch.bfloat16)
    y, h = m3.prefill(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"], 32,
                      h0=h0, x_prev=xp, B_prev=bp)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.equal(h, h0)
