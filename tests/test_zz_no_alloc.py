"""GPU test of m3_prefill_noalloc, the prefill entry point that allocates
nothing (its workspace is the library's per-GPU scratch): called through the
C ABI, its outputs equal m3_prefill's on the same inputs, on two calls in a
row, the second with a smaller input (fewer segments, so stale scratch from
the first call must not leak into it), and both are within the oracle's
tolerance."""
import ctypes

import numpy as np
import pytest

from state_space_sequence_exp_amd import inputs as I

from gpu_util import TOL, from_gpu, log, oracle_prefill, rel_l2, upload_prefill

pytestmark = pytest.mark.gpu


def _noalloc_call(g, chunk, y, hf):
    """m3_prefill_noalloc straight through the C ABI (ctypes)."""
    import torch
    import state_space_sequence_exp_amd as m3
    from state_space_sequence_exp_amd import _binding as bnd
    lib = m3.load_library()
    nb, nt, nh, nr, npd = g["x"].shape
    nn = g["B"].shape[-1]
    d = bnd.M3Dims(nb, nt, nh, npd, nn, nr)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.m3_prefill_noalloc(ctypes.byref(d), bnd.M3_BF16, chunk, p(g["x"]), p(g["dt"]),
                                p(g["A"]), p(g["lam"]), p(g["theta"]), p(g["B"]), p(g["C"]),
                                p(y), p(hf),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == bnd.M3_SUCCESS, bnd.status_string(st)


def test_noalloc_matches_prefill_two_calls():
    import torch
    import state_space_sequence_exp_amd as m3
    big = I.prefill_inputs(4, 2048, 16, 64, 64, 1, "bf16", seed=201)     # 256 segments
    small = I.prefill_inputs(1, 300, 3, 64, 64, 1, "bf16", seed=202)     # 15 segments
    for inp, chunk in ((big, 64), (small, 64)):
        log("noalloc prefill shape=%s" % (inp["x"].shape,))
        g = upload_prefill(inp)
        y_ref, h_ref = m3.prefill(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"],
                                  chunk, check=True)
        y = torch.full_like(y_ref, float("nan"))
        hf = torch.full_like(h_ref, float("nan"))
        _noalloc_call(g, chunk, y, hf)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(hf, h_ref)
        yo, ho = oracle_prefill(inp)
        ey, eh = rel_l2(from_gpu(y), yo), rel_l2(from_gpu(hf), ho)
        log("   rel_l2 vs oracle y=%.3e h=%.3e" % (ey, eh))
        assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """A shape whose workspace exceeds the scratch is refused before any HIP
    call (M3_ERR_WORKSPACE), and nothing is written."""
    import torch
    import state_space_sequence_exp_amd as m3
    need = m3.prefill_workspace_size(64, 128, 64, 64, 128, 1, 64, torch.bfloat16)
    assert need > m3._binding.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((64, 128, 64, 64), dtype=torch.bfloat16, device="cuda:0")
    B = torch.zeros((64, 128, 64, 128), dtype=torch.bfloat16, device="cuda:0")
    dt = torch.zeros((64, 128, 64), device="cuda:0")
    A = torch.zeros((64,), device="cuda:0")
    th = torch.zeros((64, 128, 64, 64), device="cuda:0")
    y = torch.full_like(x, 3.0)
    with pytest.raises(m3.M3Error) as ei:
        m3.prefill_noalloc(x, dt, A, dt, th, B, B, 64, y)
    assert ei.value.status == m3._binding.M3_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
