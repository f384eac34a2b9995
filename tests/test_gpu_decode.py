"""GPU parity of m3_decode_step against the fp64 oracle, and the
prefill -> decode hand-over."""
import numpy as np
import pytest

from state_space_sequence_exp_amd import inputs as I

from gpu_util import (TOL, from_gpu, gpu_prefill, log, oracle_prefill, oracle_threads, record_parity,
                      rel_l2, to_gpu_f32, to_gpu_storage, upload_prefill, worst_state_rel)

pytestmark = pytest.mark.gpu


def upload_ring(inp):
    dt = inp["dtype"]
    return dict(x=to_gpu_storage(inp["x_raw"], dt), B=to_gpu_storage(inp["B_raw"], dt),
                C=to_gpu_storage(inp["C_raw"], dt), dt=to_gpu_f32(inp["dt"]),
                lam=to_gpu_f32(inp["lam"]), theta=to_gpu_f32(inp["theta"]),
                A=to_gpu_f32(inp["A"]))


def run_decode(inp, steps, sel, record_steps=(), matrix_cores=False):
    """Run `steps` decode steps on the GPU over the whole batch and the oracle
    over sequences `sel`; returns (y_gpu, y_ref, h_gpu, h_ref) at the end and
    the errors of y at record_steps.  matrix_cores: through
    m3_decode_step_mfma."""
    import torch
    import oracle
    import state_space_sequence_exp_amd as m3
    K = inp["x"].shape[0]
    g = upload_ring(inp)
    h = to_gpu_f32(inp["h0"])
    h_ref = inp["h0"][sel].astype(np.float64)
    errs = []
    y = None
    for t in range(steps):
        cur, prev = t % K, (t - 1) % K
        y, h = m3.decode_step(h, g["x"][cur], g["x"][prev], g["B"][cur], g["B"][prev],
                              g["C"][cur], g["dt"][cur], g["A"], g["lam"][cur], g["theta"][cur],
                              matrix_cores=matrix_cores)
        y_ref, h_ref = oracle.decode_step(
            h_ref, inp["x"][cur][sel], inp["x"][prev][sel], inp["B"][cur][sel],
            inp["B"][prev][sel], inp["C"][cur][sel], inp["dt"][cur][sel], inp["A"],
            inp["lam"][cur][sel], inp["theta"][cur][sel], nthreads=oracle_threads())
        if t in record_steps:
            errs.append((t, rel_l2(from_gpu(y)[sel], y_ref)))
    torch.cuda.synchronize()
    return from_gpu(y)[sel], y_ref, from_gpu(h)[sel], h_ref, errs


SMALL = [
    # dtype, S, H, N, P, R, steps
    ("f32", 3, 2, 16, 16, 1, 7),
    ("f32", 2, 3, 64, 64, 2, 5),
    ("f32", 2, 2, 128, 64, 4, 9),
    ("f32", 1, 2, 30, 32, 1, 4),
    ("bf16", 3, 2, 128, 64, 4, 9),
    ("bf16", 2, 2, 64, 128, 2, 6),
    ("bf16", 2, 2, 256, 16, 1, 5),
    ("bf16", 4, 1, 128, 128, 4, 3),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "%s-s%d-h%d-n%d-p%d-r%d-k%d" % c)
def test_decode_small(case):
    dtype, S, H, N, P, R, steps = case
    inp = I.decode_inputs(S, H, N, P, R, dtype, ring=4, seed=7 + N + P)
    log("decode small %s" % (case,))
    sel = np.arange(S)
    y, y_ref, h, h_ref, _ = run_decode(inp, steps, sel)
    ey, eh = rel_l2(y, y_ref), rel_l2(h, h_ref)
    log("   rel_l2 y=%.3e h=%.3e" % (ey, eh))
    assert ey <= TOL[dtype] and eh <= TOL[dtype]


def worst_decode_y(y, y_ref):
    """Worst rel-L2 over (sequence, head) units of y [S,H,R,P]."""
    return max(rel_l2(y[s, k], y_ref[s, k]) for s in range(y.shape[0]) for k in range(y.shape[1]))


def test_decode_config4_full_batch():
    """The whole decode workload (256 sequences x 32 heads, N=128, P=64,
    R=4, bf16) for 32 steps from the seeded initial state, every unit against
    the oracle: whole-tensor and worst-unit rel-L2 of y and of the state."""
    inp = I.decode_config_inputs()
    sel = np.arange(inp["h0"].shape[0])
    log("decode config4: 32 steps, oracle on the full batch")
    y, y_ref, h, h_ref, errs = run_decode(inp, 32, sel, record_steps=(0, 15, 31))
    ey, eh = rel_l2(y, y_ref), rel_l2(h, h_ref)
    wy, wh = worst_decode_y(y, y_ref), worst_state_rel(h, h_ref)
    log("   rel_l2 y=%.3e h=%.3e worst-unit y=%.3e h=%.3e; y along the way: %s"
        % (ey, eh, wy, wh, errs))
    record_parity("decode config4 full batch, 32 steps", y=ey, h=eh, worst_y=wy, worst_h=wh,
                  tol=TOL["bf16"])
    assert max(ey, eh, wy, wh) <= TOL["bf16"]
    assert all(e <= TOL["bf16"] for _, e in errs)


def test_decode_config4_1000_steps():
    """Full batch (256 sequences x 32 heads, N=128, P=64, R=4) on the GPU for
    1000 steps; the oracle follows sequences 0-7 (all heads)."""
    inp = I.decode_config_inputs()
    sel = np.arange(8)
    log("decode config4: 1000 steps, oracle on sequences 0-7")
    y, y_ref, h, h_ref, errs = run_decode(inp, 1000, sel, record_steps=(0, 1, 2, 499, 999))
    ey, eh = rel_l2(y, y_ref), rel_l2(h, h_ref)
    wy, wh = worst_decode_y(y, y_ref), worst_state_rel(h, h_ref)
    log("   rel_l2 y=%.3e h=%.3e worst-unit y=%.3e h=%.3e; y along the way: %s"
        % (ey, eh, wy, wh, errs))
    record_parity("decode config4 sequences 0-7, 1000 steps", y=ey, h=eh, worst_y=wy,
                  worst_h=wh, tol=TOL["bf16"])
    assert max(ey, eh, wy, wh) <= TOL["bf16"]
    assert all(e <= TOL["bf16"] for _, e in errs)


@pytest.mark.parametrize("dtype,R", [("f32", 1), ("f32", 4), ("bf16", 4)])
def test_decode_lambda_zero(dtype, R):
    """lam = 0: the current input enters only through the next step's beta
    term."""
    inp = I.decode_inputs(3, 2, 64, 64, R, dtype, ring=4, seed=83 + R)
    inp["lam"][:] = 0.0
    log("decode lam=0 %s R=%d" % (dtype, R))
    sel = np.arange(3)
    y, y_ref, h, h_ref, _ = run_decode(inp, 6, sel)
    ey, eh = rel_l2(y, y_ref), rel_l2(h, h_ref)
    log("   rel_l2 y=%.3e h=%.3e" % (ey, eh))
    assert ey <= TOL[dtype] and eh <= TOL[dtype]


def test_decode_in_place_equals_out_of_place():
    import torch
    import state_space_sequence_exp_amd as m3
    inp = I.decode_inputs(4, 4, 128, 64, 4, "bf16", ring=2, seed=5)
    g = upload_ring(inp)
    h1 = to_gpu_f32(inp["h0"])
    h2 = h1.clone()
    out = torch.empty_like(h1)
    args = (g["x"][1], g["x"][0], g["B"][1], g["B"][0], g["C"][1], g["dt"][1], g["A"],
            g["lam"][1], g["theta"][1])
    ya, _ = m3.decode_step(h1, *args)                 # in place
    yb, _ = m3.decode_step(h2, *args, h_out=out)      # out of place
    torch.cuda.synchronize()
    assert torch.equal(h1, out) and torch.equal(ya, yb)


@pytest.mark.parametrize("dtype,R", [("f32", 1), ("bf16", 4)])
def test_prefill_then_decode_continues_the_sequence(dtype, R):
    """prefill(T) then k decode steps == prefill(T + k), on the GPU and vs the oracle."""
    import torch
    import state_space_sequence_exp_amd as m3
    T, k = 512, 16
    chunk = 64 if R == 1 else 32   # N=128 with R=4 at chunk 64 exceeds the LDS budget
    inp = I.prefill_inputs(2, T + k, 2, 128, 64, R, dtype, seed=61)
    g = upload_prefill(inp)
    sl = lambda t, a, b: t[:, a:b].contiguous()
    log("prefill %d then decode %d (%s, R=%d)" % (T, k, dtype, R))
    y_pre, h = m3.prefill(sl(g["x"], 0, T), sl(g["dt"], 0, T), g["A"], sl(g["lam"], 0, T),
                          sl(g["theta"], 0, T), sl(g["B"], 0, T), sl(g["C"], 0, T), chunk)
    ys = []
    for t in range(T, T + k):
        y, h = m3.decode_step(h, g["x"][:, t].contiguous(), g["x"][:, t - 1].contiguous(),
                              g["B"][:, t].contiguous(), g["B"][:, t - 1].contiguous(),
                              g["C"][:, t].contiguous(), g["dt"][:, t].contiguous(), g["A"],
                              g["lam"][:, t].contiguous(), g["theta"][:, t].contiguous())
        ys.append(y)
    torch.cuda.synchronize()
    y_dec = np.stack([from_gpu(v) for v in ys], axis=1)     # [B, k, H, R, P]
    y_full, h_full = gpu_prefill(inp, chunk, g)
    y_full, h_full = from_gpu(y_full), from_gpu(h_full)
    y_ref, h_ref = oracle_prefill(inp)
    tol = TOL[dtype]
    e1 = rel_l2(y_dec, y_full[:, T:])
    e2 = rel_l2(y_dec, y_ref[:, T:])
    e3 = rel_l2(from_gpu(h), h_ref)
    e4 = rel_l2(from_gpu(y_pre), y_ref[:, :T])
    log("   decode vs prefill %.3e, vs oracle %.3e, h %.3e, prefix y %.3e" % (e1, e2, e3, e4))
    assert max(e1, e2, e3, e4) <= tol


# ---- the matrix-core variant (m3_decode_step_mfma) --------------------------

MFMA_SMALL = [
    # dtype, S, H, N, P, R, steps
    ("f32", 2, 3, 64, 64, 2, 5),
    ("f32", 2, 2, 128, 64, 4, 9),
    ("f32", 3, 1, 16, 64, 4, 4),
    ("bf16", 3, 2, 128, 64, 4, 9),
    ("bf16", 2, 2, 48, 64, 2, 6),
    ("bf16", 1, 3, 112, 64, 4, 5),
]


@pytest.mark.parametrize("case", MFMA_SMALL, ids=lambda c: "%s-s%d-h%d-n%d-p%d-r%d-k%d" % c)
def test_decode_mfma_small(case):
    dtype, S, H, N, P, R, steps = case
    inp = I.decode_inputs(S, H, N, P, R, dtype, ring=4, seed=11 + N + P)
    log("decode mfma small %s" % (case,))
    sel = np.arange(S)
    y, y_ref, h, h_ref, _ = run_decode(inp, steps, sel, matrix_cores=True)
    ey, eh = rel_l2(y, y_ref), rel_l2(h, h_ref)
    log("   rel_l2 y=%.3e h=%.3e" % (ey, eh))
    assert ey <= TOL[dtype] and eh <= TOL[dtype]


def test_decode_mfma_config4_full_batch():
    """The matrix-core step on the whole decode workload (256 x 32 heads,
    N=128, P=64, R=4, bf16), 32 steps, every unit against the oracle, and
    against the vector kernel's result."""
    import torch
    import state_space_sequence_exp_amd as m3
    inp = I.decode_config_inputs()
    sel = np.arange(inp["h0"].shape[0])
    log("decode mfma config4: 32 steps, oracle on the full batch")
    y, y_ref, h, h_ref, errs = run_decode(inp, 32, sel, record_steps=(0, 31), matrix_cores=True)
    ey, eh = rel_l2(y, y_ref), rel_l2(h, h_ref)
    wy, wh = worst_decode_y(y, y_ref), worst_state_rel(h, h_ref)
    log("   rel_l2 y=%.3e h=%.3e worst-unit y=%.3e h=%.3e; y along the way: %s"
        % (ey, eh, wy, wh, errs))
    record_parity("decode config4 full batch, 32 steps, MFMA", y=ey, h=eh, worst_y=wy,
                  worst_h=wh, tol=TOL["bf16"])
    assert max(ey, eh, wy, wh) <= TOL["bf16"]
    # one step of both kernels from the same state: the state agrees to float
    # rounding (the products are summed in another order)
    g = upload_ring(inp)
    h0 = to_gpu_f32(inp["h0"])
    args = (g["x"][1], g["x"][0], g["B"][1], g["B"][0], g["C"][1], g["dt"][1], g["A"],
            g["lam"][1], g["theta"][1])
    ya, ha = m3.decode_step(h0, *args, h_out=torch.empty_like(h0))
    yb, hb = m3.decode_step(h0, *args, h_out=torch.empty_like(h0), matrix_cores=True)
    torch.cuda.synchronize()
    assert rel_l2(from_gpu(hb), from_gpu(ha)) <= 1e-6
    assert rel_l2(from_gpu(yb), from_gpu(ya)) <= TOL["bf16"]


def test_decode_mfma_in_place_equals_out_of_place():
    import torch
    import state_space_sequence_exp_amd as m3
    inp = I.decode_inputs(4, 4, 128, 64, 4, "bf16", ring=2, seed=6)
    g = upload_ring(inp)
    h1 = to_gpu_f32(inp["h0"])
    h2 = h1.clone()
    out = torch.empty_like(h1)
    args = (g["x"][1], g["x"][0], g["B"][1], g["B"][0], g["C"][1], g["dt"][1], g["A"],
            g["lam"][1], g["theta"][1])
    ya, _ = m3.decode_step(h1, *args, matrix_cores=True)
    yb, _ = m3.decode_step(h2, *args, h_out=out, matrix_cores=True)
    torch.cuda.synchronize()
    assert torch.equal(h1, out) and torch.equal(ya, yb)


@pytest.mark.parametrize("N,P,R", [(64, 64, 1), (64, 32, 4), (136, 64, 4), (40, 64, 2)])
def test_decode_mfma_rejects_other_shapes(N, P, R):
    """Shapes outside R in {2, 4}, P = 64, N a multiple of 16 up to 128 are
    refused before any launch."""
    import state_space_sequence_exp_amd as m3
    from state_space_sequence_exp_amd._binding import M3Error, M3_ERR_NOT_SUPPORTED
    inp = I.decode_inputs(1, 1, N, P, R, "f32", ring=2, seed=3)
    g = upload_ring(inp)
    h = to_gpu_f32(inp["h0"])
    with pytest.raises(M3Error) as ei:
        m3.decode_step(h, g["x"][1], g["x"][0], g["B"][1], g["B"][0], g["C"][1], g["dt"][1],
                       g["A"], g["lam"][1], g["theta"][1], matrix_cores=True)
    assert ei.value.status == M3_ERR_NOT_SUPPORTED
