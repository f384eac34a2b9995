"""GPU parity of the reduced forms against the fp64 oracle, through the C ABI.

lam absent means lam = 1 (the exponential-Euler rule: the update becomes
Mamba-2's h = e^{dt A} h + dt B x^T), theta absent means theta = 0 (a real
state, no rotation); both absent is the Mamba-2 recurrence.  The oracle runs
the full recurrence with lam = 1 and / or theta = 0 arrays; its reduction to
the Mamba-2 rule is pinned on the CPU (the lam = 1, theta = 0 pin).  Prefill
also checks that an absent input gives exactly (bit for bit) the result of
passing the ones / zeros explicitly.  The decode shapes of the decode-latency
sweep (batch 128, 64 heads of P = 64, N in {64, 128}, fp32 and bf16, Mamba-2 /
SISO / MIMO R = 4) run at full batch with the oracle on sampled sequences."""
import numpy as np
import pytest

from state_space_sequence_exp_amd import inputs as I

from gpu_util import (TOL, from_gpu, log, oracle_prefill, oracle_threads, rel_l2, to_gpu_f32,
                      to_gpu_storage, upload_prefill)

pytestmark = pytest.mark.gpu

# name, lam given, theta given
MODES = [("euler", False, True), ("real", True, False), ("mamba2", False, False)]


def reduced(inp, with_lam, with_theta):
    """The same inputs with lam = 1 and / or theta = 0 written out."""
    out = dict(inp)
    if not with_lam:
        out["lam"] = np.ones_like(inp["lam"])
    if not with_theta:
        out["theta"] = np.zeros_like(inp["theta"])
    return out


PREFILL = [
    # dtype, batch, T, heads, N, P, R, chunk
    ("f32", 1, 150, 2, 32, 32, 2, 32),
    ("bf16", 2, 300, 2, 64, 64, 1, 64),
    ("bf16", 1, 200, 2, 128, 64, 1, 64),
    ("bf16", 1, 130, 2, 64, 64, 4, 32),
]


@pytest.mark.parametrize("mode", MODES, ids=lambda m: m[0])
@pytest.mark.parametrize("case", PREFILL, ids=lambda c: "%s-t%d-n%d-p%d-r%d-l%d" % (
    c[0], c[2], c[4], c[5], c[6], c[7]))
def test_prefill_reduced_forms(case, mode):
    import torch
    import state_space_sequence_exp_amd as m3
    dtype, nb, T, nh, N, P, R, chunk = case
    name, with_lam, with_theta = mode
    log("prefill %s %s" % (name, case))
    inp = I.prefill_inputs(nb, T, nh, N, P, R, dtype, seed=90 + N + R)
    g = upload_prefill(inp)
    y, h = m3.prefill(g["x"], g["dt"], g["A"], g["lam"] if with_lam else None,
                      g["theta"] if with_theta else None, g["B"], g["C"], chunk)
    red = reduced(inp, with_lam, with_theta)
    y_ref, h_ref = oracle_prefill(red)
    ey, eh = rel_l2(from_gpu(y), y_ref), rel_l2(from_gpu(h), h_ref)
    log("   rel_l2 y=%.3e h=%.3e" % (ey, eh))
    assert ey <= TOL[dtype] and eh <= TOL[dtype]
    # an absent input is exactly lam = 1 / theta = 0
    y2, h2 = m3.prefill(g["x"], g["dt"], g["A"], to_gpu_f32(red["lam"]),
                        to_gpu_f32(red["theta"]), g["B"], g["C"], chunk)
    torch.cuda.synchronize()
    assert np.array_equal(from_gpu(y), from_gpu(y2)) and np.array_equal(from_gpu(h), from_gpu(h2))
    # and differs from the full recurrence (the reduced form is really taken)
    y_full, _ = oracle_prefill(inp)
    assert rel_l2(y_ref, y_full) > 10 * TOL[dtype]


def run_decode_mode(inp, steps, sel, with_lam, with_theta, matrix_cores=False):
    """`steps` decode steps over the whole batch on the GPU (lam / theta
    absent as asked; without lam no previous token is passed) and over
    sequences `sel` in the oracle with lam = 1 / theta = 0."""
    import torch
    import oracle
    import state_space_sequence_exp_amd as m3
    K = inp["x"].shape[0]
    dt_ = inp["dtype"]
    g = dict(x=to_gpu_storage(inp["x_raw"], dt_), B=to_gpu_storage(inp["B_raw"], dt_),
             C=to_gpu_storage(inp["C_raw"], dt_), dt=to_gpu_f32(inp["dt"]),
             lam=to_gpu_f32(inp["lam"]), theta=to_gpu_f32(inp["theta"]), A=to_gpu_f32(inp["A"]))
    red = reduced(inp, with_lam, with_theta)
    h = to_gpu_f32(inp["h0"])
    h_ref = inp["h0"][sel].astype(np.float64)
    y = y_ref = None
    for t in range(steps):
        cur, prev = t % K, (t - 1) % K
        y, h = m3.decode_step(h, g["x"][cur], g["x"][prev] if with_lam else None, g["B"][cur],
                              g["B"][prev] if with_lam else None, g["C"][cur], g["dt"][cur],
                              g["A"], g["lam"][cur] if with_lam else None,
                              g["theta"][cur] if with_theta else None,
                              matrix_cores=matrix_cores)
        y_ref, h_ref = oracle.decode_step(
            h_ref, red["x"][cur][sel], red["x"][prev][sel], red["B"][cur][sel],
            red["B"][prev][sel], red["C"][cur][sel], red["dt"][cur][sel], red["A"],
            red["lam"][cur][sel], red["theta"][cur][sel], nthreads=oracle_threads())
    torch.cuda.synchronize()
    return from_gpu(y)[sel], y_ref, from_gpu(h)[sel], h_ref


@pytest.mark.parametrize("mode", MODES, ids=lambda m: m[0])
@pytest.mark.parametrize("case", [("f32", 64, 1), ("f32", 128, 4), ("bf16", 64, 4),
                                  ("bf16", 128, 1)], ids=lambda c: "%s-n%d-r%d" % c)
def test_decode_reduced_forms(case, mode):
    dtype, N, R = case
    name, with_lam, with_theta = mode
    log("decode %s %s" % (name, case))
    inp = I.decode_inputs(3, 2, N, 64, R, dtype, ring=3, seed=95 + N + R)
    sel = np.arange(3)
    y, y_ref, h, h_ref = run_decode_mode(inp, 6, sel, with_lam, with_theta)
    ey, eh = rel_l2(y, y_ref), rel_l2(h, h_ref)
    log("   rel_l2 y=%.3e h=%.3e" % (ey, eh))
    assert ey <= TOL[dtype] and eh <= TOL[dtype]


@pytest.mark.parametrize("mode", MODES, ids=lambda m: m[0])
@pytest.mark.parametrize("case", [("f32", 128, 4), ("bf16", 64, 2)], ids=lambda c: "%s-n%d-r%d" % c)
def test_decode_mfma_reduced_forms(case, mode):
    """The reduced forms through the matrix-core decode step."""
    dtype, N, R = case
    name, with_lam, with_theta = mode
    log("decode mfma %s %s" % (name, case))
    inp = I.decode_inputs(3, 2, N, 64, R, dtype, ring=3, seed=96 + N + R)
    sel = np.arange(3)
    y, y_ref, h, h_ref = run_decode_mode(inp, 6, sel, with_lam, with_theta, matrix_cores=True)
    ey, eh = rel_l2(y, y_ref), rel_l2(h, h_ref)
    log("   rel_l2 y=%.3e h=%.3e" % (ey, eh))
    assert ey <= TOL[dtype] and eh <= TOL[dtype]


# the decode-latency sweep: (variant, R, lam given, theta given)
SWEEP = [("mamba2", 1, False, False), ("siso", 1, True, True), ("mimo", 4, True, True)]


@pytest.mark.parametrize("variant", SWEEP, ids=lambda v: v[0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [64, 128])
def test_decode_sweep_shapes_full_batch(N, dtype, variant):
    """128 sequences x 64 heads (P = 64) on the GPU for 3 steps; the oracle
    follows sequences 0-3 (all heads)."""
    name, R, with_lam, with_theta = variant
    log("decode sweep %s N=%d %s" % (name, N, dtype))
    inp = I.decode_inputs(128, 64, N, 64, R, dtype, ring=2, seed=97 + N + R)
    sel = np.arange(4)
    y, y_ref, h, h_ref = run_decode_mode(inp, 3, sel, with_lam, with_theta)
    ey, eh = rel_l2(y, y_ref), rel_l2(h, h_ref)
    log("   rel_l2 y=%.3e h=%.3e" % (ey, eh))
    assert ey <= TOL[dtype] and eh <= TOL[dtype]
