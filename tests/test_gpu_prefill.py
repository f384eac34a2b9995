"""GPU parity of m3_prefill against the fp64 oracle (through the C ABI).

Tolerance: relative L2 over a whole output tensor <= 1e-4 for float32
inputs and <= 2e-2 for bfloat16 inputs, separately for y and for the final
state (the worst per-(b,h) unit is printed too)."""
import numpy as np
import pytest

from state_space_sequence_exp_amd import inputs as I

from gpu_util import (TOL, counter_words, from_gpu, gpu_prefill, log, oracle_prefill, record_parity,
                      rel_l2, upload_prefill, worst_state_rel, worst_unit_rel)

pytestmark = pytest.mark.gpu


def check_prefill(inp, chunk, units=None, label=""):
    """GPU prefill vs the oracle: whole-tensor rel-L2 of y and of the final
    state, and (over every (b, h) unit) the worst unit of each, all within
    the dtype's tolerance."""
    log("prefill %s chunk=%d shape=%s dtype=%s" % (label, chunk, inp["x"].shape, inp["dtype"]))
    y, hf = gpu_prefill(inp, chunk)
    y, hf = from_gpu(y), from_gpu(hf)
    y_ref, h_ref = oracle_prefill(inp, units=units)
    if units is not None:
        nh = inp["x"].shape[2]
        sel = [divmod(u, nh) for u in units]
        y = np.stack([y[b, :, h] for b, h in sel])[:, :, None]
        y_ref = np.stack([y_ref[b, :, h] for b, h in sel])[:, :, None]
        hf = np.stack([hf[b, h] for b, h in sel])[:, None]
        h_ref = np.stack([h_ref[b, h] for b, h in sel])[:, None]
    ey, eh = rel_l2(y, y_ref), rel_l2(hf, h_ref)
    wy = worst_unit_rel(y.reshape(y.shape[:3] + (-1,)), y_ref.reshape(y.shape[:3] + (-1,)))
    wh = worst_state_rel(hf, h_ref)
    tol = TOL[inp["dtype"]]
    log("   rel_l2 y=%.3e h=%.3e worst-unit y=%.3e h=%.3e (tol %.0e)" % (ey, eh, wy, wh, tol))
    if label.startswith("config"):
        record_parity("prefill %s %s" % (label, inp["dtype"]), y=ey, h=eh, worst_y=wy, worst_h=wh,
                      tol=tol)
    assert np.isfinite(y).all() and np.isfinite(hf).all()
    assert ey <= tol and eh <= tol
    assert wy <= tol and wh <= tol
    return y, hf


def test_config0_full():
    cfg = I.WORKLOADS[0]
    check_prefill(I.config_inputs(0), cfg.chunk, label="config0")


SMALL = [
    # dtype, B, T, H, N, P, R, chunk
    ("f32", 1, 1, 1, 16, 16, 1, 16),
    ("f32", 2, 100, 3, 16, 16, 1, 16),
    ("f32", 2, 77, 2, 32, 32, 2, 32),
    ("f32", 1, 50, 2, 64, 64, 4, 16),
    ("f32", 1, 130, 1, 16, 128, 1, 64),
    ("f32", 1, 257, 2, 128, 64, 1, 64),
    ("f32", 1, 200, 1, 64, 64, 1, 128),
    ("bf16", 2, 300, 3, 64, 64, 1, 64),
    ("bf16", 1, 200, 2, 128, 64, 1, 64),
    ("bf16", 1, 150, 2, 64, 64, 4, 64),
    ("bf16", 2, 65, 2, 32, 16, 2, 32),
    ("bf16", 1, 90, 2, 256, 32, 1, 32),
    ("bf16", 1, 33, 1, 64, 128, 2, 16),
    ("bf16", 1, 700, 1, 64, 64, 1, 128),
    # the bf16 R = 1 kernels with N fixed at the head dimensions besides 64
    # (N = 64: the split output pass at P = 16 and 32; N = 128, which has
    # its own source file and scheduling strategy, at P = 16 and 32; N P is
    # at most 8192)
    ("bf16", 1, 120, 2, 64, 32, 1, 64),
    ("bf16", 1, 90, 1, 64, 16, 1, 64),
    ("bf16", 1, 150, 2, 128, 32, 1, 64),
    ("bf16", 1, 100, 1, 128, 16, 1, 32),
    # state sizes that are not powers of two take the kernel with N read at
    # run time, whose tile counts do not divide evenly over the waves
    ("f32", 1, 150, 2, 48, 64, 1, 64),
    ("f32", 2, 70, 1, 80, 32, 2, 32),
    ("f32", 1, 60, 1, 224, 16, 1, 32),
    ("bf16", 1, 200, 2, 96, 64, 1, 64),
    ("bf16", 1, 130, 2, 192, 32, 1, 32),
    ("bf16", 1, 90, 1, 160, 16, 4, 16),
    ("bf16", 2, 100, 1, 224, 16, 2, 16),
    # workgroups draw tickets from one counter per class, the classes the
    # largest power of two up to 8 dividing batch * heads: 8 (both kernels),
    # 4 and 1, every sequence cut into several one-chunk segments
    ("bf16", 2, 300, 4, 64, 64, 1, 64),
    ("f32", 2, 200, 4, 32, 32, 1, 32),
    ("bf16", 3, 250, 4, 64, 64, 1, 64),
    ("bf16", 1, 300, 5, 128, 64, 1, 64),
    # N = 128, P <= 64, 64-token chunks: the output pass hands the scores of
    # query blocks 2 and 3 against the first key pair between waves (P = 16,
    # one p-tile a unit; a ragged last chunk of 62 tokens)
    ("bf16", 1, 190, 1, 128, 16, 1, 64),
    # sixteen query blocks a chunk (chunk x R = 256) with P <= 64: one unit
    # per query block, dealt unevenly between the waves that share a SIMD
    ("f32", 1, 150, 1, 32, 32, 4, 64),
    ("bf16", 1, 300, 2, 64, 32, 4, 64),
    ("bf16", 1, 130, 1, 64, 16, 4, 64),
    # bfloat16, R = 1, N = P = 64, 64-token chunks: the single-pass kernel
    # with segments of 5 chunks (the last chunk ragged), of 7, and of 4 over
    # four groups of segments; and, past 8 chunks a segment, the two-pass
    # token-lane kernel (32)
    ("bf16", 4, 1263, 16, 64, 64, 1, 64),
    ("bf16", 4, 1762, 16, 64, 64, 1, 64),
    ("bf16", 2, 6370, 4, 64, 64, 1, 64),
    ("bf16", 1, 8192, 64, 64, 64, 1, 64),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "%s-b%d-t%d-h%d-n%d-p%d-r%d-l%d" % c)
def test_small_shapes(case):
    dtype, b, t, h, n, p, r, chunk = case
    inp = I.prefill_inputs(b, t, h, n, p, r, dtype, seed=100 + t)
    check_prefill(inp, chunk, label="small")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_sweep_and_invariance(dtype):
    inp = I.prefill_inputs(2, 500, 2, 64, 64, 1, dtype, seed=21)
    ys = {}
    for chunk in (16, 32, 64, 128):
        ys[chunk], _ = check_prefill(inp, chunk, label="sweep")
    for chunk in (16, 32, 128):
        d = rel_l2(ys[chunk], ys[64])
        log("   chunk %d vs 64: %.3e" % (chunk, d))
        assert d <= (2e-5 if dtype == "f32" else 1e-2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_slow_decay_exposes_inter_chunk_path(dtype):
    """A = -exp(U(-8,-5)): the state survives many chunks."""
    inp = I.prefill_inputs(1, 1000, 2, 64, 64, 2, dtype, seed=31, a_range=(-8.0, -5.0))
    check_prefill(inp, 64, label="slow-decay")


@pytest.mark.parametrize("b,t,h", [(4, 2048, 16), (4, 1263, 16), (2, 6370, 4)])
def test_slow_decay_single_pass_segments(b, t, h):
    """The single-pass kernel (bfloat16, R = 1, N = P = 64, chunk 64) with
    segments of 8, 5 and 4 chunks under slow decay, so that every segment's
    outputs depend on its entry state, which reaches them only through the
    correction after the chain."""
    inp = I.prefill_inputs(b, t, h, 64, 64, 1, "bf16", seed=33 + t, a_range=(-8.0, -5.0))
    check_prefill(inp, 64, label="slow-decay-single-pass")


@pytest.mark.parametrize("dtype,R,chunk", [("f32", 1, 64), ("f32", 4, 32), ("bf16", 1, 64),
                                           ("bf16", 4, 64)])
def test_lambda_zero_extreme(dtype, R, chunk):
    """lam = 0: gamma vanishes and each input enters only through the next
    token's beta term (the previous-input half of the trapezoid)."""
    inp = I.prefill_inputs(2, 300, 2, 64, 64, R, dtype, seed=71 + R)
    inp["lam"][:] = 0.0
    check_prefill(inp, chunk, label="lam=0")


def test_parity_construction_long():
    """theta = pi * bit, A = 0, dt = 1, lam = 1, one seeded input: the state's
    sign follows the parity of the bits over 4096 steps."""
    T, N, P = 4096, 16, 16
    rng = np.random.default_rng(41)
    bits = rng.integers(0, 2, T)
    inp = I.prefill_inputs(1, T, 1, N, P, 1, "f32", seed=41)
    for k in ("x", "x_raw"):
        inp[k][:, 1:] = 0.0
    inp["dt"][:] = 1.0
    inp["lam"][:] = 1.0
    inp["A"][:] = 0.0
    inp["theta"][0, :, 0, :] = (np.pi * bits)[:, None].astype(np.float32)
    y, hf = check_prefill(inp, 64, label="parity")
    # closed form: the seed rotated by the sum of the float32 angles after step 0
    # (float32 pi differs from pi by 8.7e-8, which thousands of flips resolve)
    seed = np.outer(inp["B"][0, 0, 0, 0].astype(np.float64), inp["x"][0, 0, 0, 0])
    total = float(np.float32(np.pi)) * bits[1:].sum()
    c, s = np.cos(total), np.sin(total)
    expect = np.empty_like(seed)
    expect[0::2] = c * seed[0::2] - s * seed[1::2]
    expect[1::2] = s * seed[0::2] + c * seed[1::2]
    sign = (-1.0) ** (bits[1:].sum())
    assert rel_l2(expect, sign * seed) < 1e-3      # the parity pattern itself
    assert rel_l2(hf[0, 0], expect) < 1e-5


@pytest.mark.parametrize("index", [1, 2, 3])
def test_full_config_whole_tensor(index):
    """Full-size configuration in the launch configuration the benchmark
    times, against the oracle over every (b, h) unit and every token: the
    tolerance holds for the whole y and final-state tensors and for the worst
    unit of each."""
    cfg = I.WORKLOADS[index]
    check_prefill(I.config_inputs(index), cfg.chunk, label="config%d" % index)


@pytest.mark.parametrize("shape", [(2, 640, 4, 64, 64, 4), (4, 2048, 16, 64, 64, 1),
                                   (1, 1000, 8, 128, 64, 1)],
                         ids=["mimo", "single-pass", "n128-handover"])
def test_repeatable_bitwise(shape):
    """Repeated calls give the same bits: the chain composes every entry in
    one fixed order, and the hand-overs of scores between waves (the single
    pass's, and the N = 128 output pass's) are complete before they are
    read."""
    inp = I.prefill_inputs(*shape, "bf16", seed=51)
    g = upload_prefill(inp)
    y1, h1 = gpu_prefill(inp, 64, g)
    y2, h2 = gpu_prefill(inp, 64, g, calls=3)   # one workspace, three calls
    assert np.array_equal(from_gpu(y1), from_gpu(y2))
    assert np.array_equal(from_gpu(h1), from_gpu(h2))


def test_workspace_reused_across_shapes():
    """The kernel returns the workspace's chain counters to zero, so one
    zero-filled buffer serves successive calls of different shapes."""
    import torch
    import state_space_sequence_exp_amd as m3
    big = I.prefill_inputs(2, 900, 3, 64, 64, 1, "bf16", seed=61)
    small = I.prefill_inputs(1, 300, 2, 64, 32, 2, "bf16", seed=62)
    gb, gs = upload_prefill(big), upload_prefill(small)
    need = max(m3.prefill_workspace_size(2, 900, 3, 64, 64, 1, 64, gb["x"].dtype),
               m3.prefill_workspace_size(1, 300, 2, 32, 64, 2, 32, gs["x"].dtype))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    outs = []
    for g, chunk in ((gb, 64), (gs, 32), (gb, 64), (gs, 32)):
        outs.append(m3.prefill(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"],
                               chunk, workspace=ws))
    torch.cuda.synchronize()
    for (y, h), inp in ((outs[2], big), (outs[3], small)):
        y_ref, h_ref = oracle_prefill(inp)
        assert rel_l2(from_gpu(y), y_ref) <= TOL["bf16"]
        assert rel_l2(from_gpu(h), h_ref) <= TOL["bf16"]
    assert np.array_equal(from_gpu(outs[0][0]), from_gpu(outs[2][0]))
    assert np.array_equal(from_gpu(outs[1][0]), from_gpu(outs[3][0]))
    nw = max(counter_words(2, 900, 3, 64), counter_words(1, 300, 2, 32))
    assert not ws[:4 * nw].view(torch.int32).cpu().numpy().any()


@pytest.mark.parametrize("n", [32, 64])
def test_dirty_counters_reported(n):
    """A workspace whose class-0 ticket word is not zero on entry makes every
    workgroup of that class skip its segment and raise the error word (2);
    the counters are still returned to zero, so the next call (error word
    cleared) is correct.  N = 64 takes the single-pass kernel."""
    import torch
    import state_space_sequence_exp_amd as m3
    inp = I.prefill_inputs(1, 200, 2, n, 64, 1, "bf16", seed=63)
    g = upload_prefill(inp)
    need = m3.prefill_workspace_size(1, 200, 2, 64, n, 1, 64, g["x"].dtype)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    words = ws[:4 * counter_words(1, 200, 2, 64)].view(torch.int32)
    words[0] = 1 << 20                   # a ticket far past the grid
    m3.prefill(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"], 64, workspace=ws)
    w = words.cpu().numpy()
    assert w[1] == 2 and w[0] == 0 and w[2] == 0 and not w[4:].any(), w
    with pytest.raises(m3.M3Error):
        m3.prefill(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"], 64,
                   workspace=ws, check=True)
    assert m3.prefill_workspace_error(ws, clear=True) == 2
    assert m3.prefill_workspace_error(ws) == 0
    y, h = m3.prefill(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"], 64,
                      workspace=ws, check=True)
    assert not words.cpu().numpy().any()
    y_ref, h_ref = oracle_prefill(inp)
    assert rel_l2(from_gpu(y), y_ref) <= TOL["bf16"]
    assert rel_l2(from_gpu(h), h_ref) <= TOL["bf16"]


def test_empty_and_optional_outputs():
    import torch
    import state_space_sequence_exp_amd as m3
    inp = I.prefill_inputs(2, 0, 2, 32, 16, 1, "bf16", seed=3)
    g = upload_prefill(inp)
    hf = torch.full((2, 2, 32, 16), 7.0, device="cuda:0")
    y, hf2 = m3.prefill(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"], 32,
                        h_final=hf)
    torch.cuda.synchronize()
    assert y.numel() == 0 and float(hf.abs().max()) == 0.0
    inp = I.prefill_inputs(1, 40, 1, 32, 16, 1, "bf16", seed=4)
    g = upload_prefill(inp)
    y, hf = m3.prefill(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"], 32,
                       want_h_final=False)
    assert hf is None
    y_ref, _ = oracle_prefill(inp)
    assert rel_l2(from_gpu(y), y_ref) < TOL["bf16"]
