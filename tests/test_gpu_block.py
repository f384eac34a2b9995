"""GPU parity of the block-side passes (m3_block_prepass / m3_block_postpass)
against the fp64 oracle (oracle/block.py), through the C ABI.

Tolerances, from the arithmetic: a bfloat16 output is the fp32 result
rounded to nearest even, at most 2^-8 relative per element, so rel-L2 over a
tensor is at most 2^-8 (taken as 4e-3); float32 outputs carry only the fp32
sum of squares over N <= 256 channels and a reciprocal root, far under 1e-5.
The whole block -- pre-pass, prefill, post-pass -- is held to the prefill
tolerances."""
import numpy as np
import pytest

from state_space_sequence_exp_amd import inputs as I

from gpu_util import (TOL, from_gpu, log, oracle_threads, rel_l2, to_gpu_f32, to_gpu_storage)

pytestmark = pytest.mark.gpu

PASS_TOL = {"f32": 1e-5, "bf16": 4e-3}


def upload_block(inp):
    dt = inp["dtype"]
    g = {k: to_gpu_storage(inp[k + "_raw"], dt) for k in ("x", "B", "C")}
    for k in ("norm_B", "norm_C", "bias_B", "bias_C", "up", "down"):
        g[k] = to_gpu_f32(inp[k])
    return g


def oracle_pre(inp, eps):
    from oracle import block
    return block.block_prepass(inp["x"], inp["B"], inp["C"], inp["norm_B"], inp["norm_C"],
                               inp["bias_B"], inp["bias_C"], inp["up"], eps)


CASES = [
    # dtype, batch, T, heads, N, P, R
    ("f32", 2, 37, 3, 64, 64, 1),
    ("f32", 1, 20, 2, 256, 16, 4),
    ("bf16", 2, 100, 3, 64, 64, 1),
    ("bf16", 1, 50, 2, 128, 64, 4),
    ("bf16", 3, 9, 2, 16, 128, 2),
    ("bf16", 1, 33, 1, 256, 32, 1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-b%d-t%d-h%d-n%d-p%d-r%d" % c)
def test_prepass_and_postpass(case):
    import state_space_sequence_exp_amd as m3
    dtype, nb, T, nh, N, P, R = case
    log("block passes %s" % (case,))
    inp = I.block_inputs(nb, T, nh, N, P, R, dtype, seed=100 + N + P + R)
    g = upload_block(inp)
    eps = 1e-5
    X, Bt, Ct = m3.block_prepass(g["x"], g["B"], g["C"], g["norm_B"], g["norm_C"], g["bias_B"],
                                 g["bias_C"], g["up"], eps)
    Xr, Br, Cr = oracle_pre(inp, eps)
    errs = [rel_l2(from_gpu(X), Xr), rel_l2(from_gpu(Bt), Br), rel_l2(from_gpu(Ct), Cr)]
    log("   pre-pass rel_l2 X=%.2e B=%.2e C=%.2e" % tuple(errs))
    assert max(errs) <= PASS_TOL[dtype]
    # post-pass on an independent y of the SSM's output shape
    from oracle import block
    y32 = np.random.default_rng(7).standard_normal((nb, T, nh, R, P)).astype(np.float32)
    yv, yraw = I._store(y32, dtype)
    out = m3.block_postpass(to_gpu_storage(yraw, dtype), g["down"])
    e = rel_l2(from_gpu(out), block.block_postpass(yv, inp["down"]))
    log("   post-pass rel_l2 %.2e" % e)
    assert e <= PASS_TOL[dtype]


def test_in_place_and_empty():
    import torch
    import state_space_sequence_exp_amd as m3
    inp = I.block_inputs(2, 40, 2, 64, 64, 1, "bf16", seed=111)
    g = upload_block(inp)
    X, Bt, Ct = m3.block_prepass(g["x"], g["B"], g["C"], g["norm_B"], g["norm_C"], g["bias_B"],
                                 g["bias_C"], g["up"], 1e-6)
    x2, B2, C2 = g["x"].clone(), g["B"].clone(), g["C"].clone()
    X2, Bo, Co = m3.block_prepass(x2, B2, C2, g["norm_B"], g["norm_C"], g["bias_B"], g["bias_C"],
                                  g["up"], 1e-6, x_out=x2.view(2, 40, 2, 1, 64), B_out=B2,
                                  C_out=C2)
    torch.cuda.synchronize()
    assert torch.equal(X, X2) and torch.equal(Bt, Bo) and torch.equal(Ct, Co)
    e = I.block_inputs(2, 0, 2, 64, 64, 1, "bf16", seed=112)
    ge = upload_block(e)
    X, Bt, Ct = m3.block_prepass(ge["x"], ge["B"], ge["C"], ge["norm_B"], ge["norm_C"],
                                 ge["bias_B"], ge["bias_C"], ge["up"], 1e-6)
    assert X.numel() == 0 and Bt.numel() == 0


@pytest.mark.parametrize("dtype,R", [("bf16", 1), ("bf16", 4), ("f32", 2)])
def test_whole_block_against_oracle(dtype, R):
    """pre-pass -> prefill -> post-pass against the same chain in the oracle
    (fp64 throughout; the GPU rounds X, B~, C~ and y to the storage type)."""
    import oracle
    import state_space_sequence_exp_amd as m3
    from oracle import block
    nb, T, nh, N, P = 2, 200, 2, 64, 64
    log("whole block %s R=%d" % (dtype, R))
    inp = I.block_inputs(nb, T, nh, N, P, R, dtype, seed=120 + R)
    ssm = I.prefill_inputs(nb, T, nh, N, P, R, dtype, seed=121 + R)
    g = upload_block(inp)
    X, Bt, Ct = m3.block_prepass(g["x"], g["B"], g["C"], g["norm_B"], g["norm_C"], g["bias_B"],
                                 g["bias_C"], g["up"], 1e-6)
    y, h = m3.prefill(X, to_gpu_f32(ssm["dt"]), to_gpu_f32(ssm["A"]), to_gpu_f32(ssm["lam"]),
                      to_gpu_f32(ssm["theta"]), Bt, Ct, 64)
    out = m3.block_postpass(y, g["down"])
    Xr, Br, Cr = block.block_prepass(inp["x"], inp["B"], inp["C"], inp["norm_B"],
                                     inp["norm_C"], inp["bias_B"], inp["bias_C"], inp["up"], 1e-6)
    yr, hr = oracle.prefill(Xr, ssm["dt"], ssm["A"], ssm["lam"], ssm["theta"], Br, Cr,
                            nthreads=oracle_threads())
    outr = block.block_postpass(yr, inp["down"])
    eo, eh = rel_l2(from_gpu(out), outr), rel_l2(from_gpu(h), hr)
    log("   rel_l2 out=%.2e h=%.2e" % (eo, eh))
    # fp32 inputs: the oracle sees the pre-pass's fp32 rounding only
    assert eo <= TOL[dtype] and eh <= TOL[dtype]


@pytest.mark.parametrize("R", [1, 4])
def test_bench_shapes_sampled(R):
    """The bench shapes (batch 4, T 2048 / 4096, 16 heads, N = P = 64, bf16)
    at full size; the oracle checks sampled token rows."""
    import state_space_sequence_exp_amd as m3
    T = 2048 if R == 1 else 4096
    log("block passes at bench size R=%d" % R)
    inp = I.block_inputs(4, T, 16, 64, 64, R, "bf16", seed=130 + R)
    g = upload_block(inp)
    X, Bt, Ct = m3.block_prepass(g["x"], g["B"], g["C"], g["norm_B"], g["norm_C"], g["bias_B"],
                                 g["bias_C"], g["up"], 1e-6)
    rng = np.random.default_rng(131)
    bs, ts = rng.integers(0, 4, 64), rng.integers(0, T, 64)
    sub = {k: inp[k][bs, ts][:, None] for k in ("x", "B", "C")}
    sub.update({k: inp[k] for k in ("norm_B", "norm_C", "bias_B", "bias_C", "up")})
    Xr, Br, Cr = oracle_pre(sub, 1e-6)
    import torch
    ib, it = torch.as_tensor(bs, device=X.device), torch.as_tensor(ts, device=X.device)
    Xg, Bg, Cg = (from_gpu(t[ib, it])[:, None] for t in (X, Bt, Ct))
    errs = [rel_l2(Xg, Xr), rel_l2(Bg, Br), rel_l2(Cg, Cr)]
    log("   sampled rel_l2 X=%.2e B=%.2e C=%.2e" % tuple(errs))
    assert max(errs) <= PASS_TOL["bf16"]
