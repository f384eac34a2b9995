"""Helpers shared by the GPU tests: upload seeded inputs, run the GPU path
through the C ABI binding, run the oracle on the same values, compare."""
from __future__ import annotations

import os
import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


def to_gpu_storage(raw, dtype):
    """numpy storage array (float32 or uint16 bf16 bits) -> device tensor."""
    torch, dev = torch_dev()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32))
    return t.to(dev)


def to_gpu_f32(a):
    torch, dev = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def from_gpu(t):
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64)


def upload_prefill(inp):
    return dict(
        x=to_gpu_storage(inp["x_raw"], inp["dtype"]),
        B=to_gpu_storage(inp["B_raw"], inp["dtype"]),
        C=to_gpu_storage(inp["C_raw"], inp["dtype"]),
        dt=to_gpu_f32(inp["dt"]), lam=to_gpu_f32(inp["lam"]),
        theta=to_gpu_f32(inp["theta"]), A=to_gpu_f32(inp["A"]))


def prefill_grid(nb, nt, nh, chunk):
    """Workgroups (segments) of one prefill call, by the rule the workspace
    layout documents: K = clamp(ceil(nC * units / 256), 1, nC) chunks per
    segment, units * ceil(nC / K) segments."""
    units = nb * nh
    nc = max(1, -(-nt // chunk))
    k = min(nc, max(1, -(-(nc * units) // 256)))
    return units * (-(-nc // k))


def counter_words(nb, nt, nh, chunk):
    """int32 words of the workspace's chain counters: 256 (the ticket
    counters, the error word and the finished-workgroup count), then one
    status word per workgroup."""
    return 256 + prefill_grid(nb, nt, nh, chunk)


def gpu_prefill(inp, chunk, dev_inp=None, calls=1):
    """Prefill through the C ABI with an explicit zero-filled workspace (reused
    for `calls` calls), then check the workspace's chain counters: the kernel
    returned them to zero and no wait timed out."""
    import torch
    import state_space_sequence_exp_amd as m3
    g = dev_inp or upload_prefill(inp)
    nb, nt, nh, nr, npd = g["x"].shape
    nn = g["B"].shape[-1]
    need = m3.prefill_workspace_size(nb, nt, nh, npd, nn, nr, chunk, g["x"].dtype)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=g["x"].device)
    for _ in range(calls):
        y, hf = m3.prefill(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"], chunk,
                           workspace=ws)
    if need > 0:
        err = m3.prefill_workspace_error(ws)
        assert err == 0, "error word set: %d" % err
        words = ws[:4 * counter_words(nb, nt, nh, chunk)].view(torch.int32).cpu().numpy()
        assert not words.any(), "chain counters not reset: %s" % words
    return y, hf


def oracle_prefill(inp, units=None):
    import oracle
    return oracle.prefill(inp["x"], inp["dt"], inp["A"], inp["lam"], inp["theta"], inp["B"],
                          inp["C"], units=units, nthreads=oracle_threads())


def oracle_threads():
    """Host threads for the oracle: the cores this process may run on, at
    most 16 (the CPU share that goes with one GPU on the test machines)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def rel_l2(a, ref):
    a = np.asarray(a, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    return float(np.linalg.norm(a - ref) / max(np.linalg.norm(ref), 1e-300))


def worst_unit_rel(y, y_ref):
    """Worst rel-L2 over (b, h) units of a [B,T,H,...] output."""
    nb, _, nh = y.shape[:3]
    return max(rel_l2(y[b, :, h], y_ref[b, :, h]) for b in range(nb) for h in range(nh))


def worst_state_rel(h, h_ref):
    """Worst rel-L2 over (b, h) units of a [B,H,N,P] state (0 where the
    reference state is exactly zero and so is the result)."""
    nb, nh = h.shape[:2]
    worst = 0.0
    for b in range(nb):
        for k in range(nh):
            den = np.linalg.norm(h_ref[b, k])
            num = np.linalg.norm(h[b, k] - h_ref[b, k])
            worst = max(worst, num / den if den > 0 else (0.0 if num == 0 else np.inf))
    return float(worst)


# parity results of this session, printed in the terminal summary (conftest)
PARITY = []


def record_parity(label, **errs):
    PARITY.append((label, errs))


def log(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()
