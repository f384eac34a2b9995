#!/usr/bin/env python3
"""Benchmark of libm3ssm on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints ONE JSON line.  The headline `value` is SISO chunked-prefill
throughput (tokens/s, a token = one position of one sequence through all
heads of the layer) on the SISO prefill workload (batch 4, T=2048, 16 heads,
N=64, P=64, R=1, bf16 x/B/C, chunk 64): each timed step is one m3_prefill
call (all prefill kernels) on inputs already resident in HBM, with a 512 MB
scratch write between steps so that the 256 MB last-level cache (MALL) holds
none of the step's data, timed with HIP events on the stream the kernels run
on.  The same line carries, measured in the same run:

  roofline      the prefill path against the HBM roofline (algorithmic bytes
                per call / measured call duration, peak 8 TB/s), also as a
                fraction of the measured copy bandwidth
  cpu_baseline  the fp64 oracle on the host cores for the same workload
  device_anchors  this GPU's measured copy bandwidth (512 MiB) and bf16
                GEMM rate, beside the published peaks
  secondary     the tiny fp32 workload (latency), MIMO R=4 prefill (B4 T4096
                H16 N64 P64), long-context SISO prefill (B1 T16384 H64 N128
                P64) and the decode step (256 sequences x 32 heads, N128 P64
                R4; us/step and HBM GB/s with its own roofline), each with
                the oracle's CPU baseline; the decode-latency sweep, the
                block-side passes and the backward

Inputs follow the seeded recipe of state_space_sequence_exp_amd.inputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
METRIC = "SSM prefill tokens/s (SISO, MIMO R=4); decode µs/step and HBM GB/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def kernel_source_hash() -> str:
    d = os.path.join(ROOT, "state_space_sequence_exp_amd", "csrc")
    h = hashlib.sha256()
    files = []
    for dirpath, _, names in os.walk(d):
        files += [os.path.relpath(os.path.join(dirpath, n), d) for n in names]
    for name in sorted(files):
        with open(os.path.join(d, name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(key: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = t.get(key)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


# ---------------------------------------------------------------------------
def prefill_bytes(cfg) -> int:
    es = 2 if cfg.dtype == "bf16" else 4
    tokhead = cfg.batch * cfg.seqlen * cfg.nheads
    return (tokhead * cfg.R * cfg.P * es * 2          # x in, y out
            + tokhead * cfg.R * cfg.N * es * 2        # B, C
            + tokhead * 4 * 2                         # dt, lam
            + tokhead * (cfg.N // 2) * 4              # theta
            + cfg.nheads * 4                          # A
            + cfg.batch * cfg.nheads * cfg.N * cfg.P * 4)  # h_final


def prefill_flops(cfg) -> int:
    tokhead = cfg.batch * cfg.seqlen * cfg.nheads
    return tokhead * (2 * cfg.chunk * cfg.R * cfg.R * (cfg.N + cfg.P) + 4 * cfg.N * cfg.P * cfg.R)


def decode_bytes(cfg) -> int:
    es = 2 if cfg.dtype == "bf16" else 4
    per = (2 * cfg.N * cfg.P * 4 + 2 * cfg.R * cfg.P * es + 3 * cfg.R * cfg.N * es
           + (cfg.N // 2) * 4 + 8 + cfg.R * cfg.P * es)
    return cfg.batch * cfg.nheads * per + cfg.nheads * 4


def flush_mall(scratch):
    """Evict the last-level cache (MALL, 256 MB) before a cold timed call:
    write a 512 MB scratch buffer, then read it back, so the cache holds only
    clean scratch lines -- the dirty lines of the write are written back
    here, not during the timed call."""
    scratch.fill_(1.0)
    scratch.sum()


def decode_mode_bytes(S, H, N, P, R, es, trap, rot) -> int:
    """Algorithmic bytes of one decode step: the state read and written, the
    token's inputs (the previous token's x and B and lam only for the
    trapezoid rule, theta only with rotation) and y."""
    per = (2 * N * P * 4 + R * P * es + 2 * R * N * es + 4 + R * P * es
           + (R * P * es + R * N * es + 4 if trap else 0) + ((N // 2) * 4 if rot else 0))
    return S * H * per + H * 4


# decode-latency sweep: batch 128, 64 heads of P = 64 (a 1.5B model's layer,
# d_inner 4096), state size 64 or 128, fp32 or bf16 inputs; Mamba-2 (the
# exponential-Euler rule on a real state), Mamba-3 SISO and MIMO rank 4
SWEEP = [("mamba2", 1, False, False), ("mamba3_siso", 1, True, True),
         ("mamba3_mimo_r4", 4, True, True)]


def decode_sweep(steps, log):
    """Per-step decode latency for each sweep point: 'cold' steps each
    preceded by a MALL flush (the state comes from HBM, as in a
    model whose other layers evict it) and back-to-back steps."""
    import numpy as np
    import torch
    import state_space_sequence_exp_amd as m3
    from state_space_sequence_exp_amd import inputs as I
    S, H, P = 128, 64, 64
    scratch = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda:0")
    rows = []
    for N in (64, 128):
        for dtype in ("f32", "bf16"):
            for name, R, trap, rot in SWEEP:
                log("decode sweep %s N=%d %s" % (name, N, dtype))
                inp = I.decode_inputs(S, H, N, P, R, dtype, ring=2, seed=97 + N + R)
                g = upload(inp)
                del inp
                h, y = g["h0"], None

                def step(t):
                    cur, prev = t % 2, (t - 1) % 2
                    return m3.decode_step(h, g["x"][cur], g["x"][prev] if trap else None,
                                          g["B"][cur], g["B"][prev] if trap else None,
                                          g["C"][cur], g["dt"][cur], g["A"],
                                          g["lam"][cur] if trap else None,
                                          g["theta"][cur] if rot else None, y=y)
                y, _ = step(0)
                for t in range(3):
                    step(t)
                torch.cuda.synchronize()
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(steps)]
                for t, (s0, e0) in enumerate(evs):
                    flush_mall(scratch)
                    s0.record()
                    step(t)
                    e0.record()
                torch.cuda.synchronize()
                cold = float(np.median([s0.elapsed_time(e0) for s0, e0 in evs])) * 1e3
                s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s0.record()
                for t in range(steps):
                    step(t)
                e0.record()
                torch.cuda.synchronize()
                b2b = s0.elapsed_time(e0) / steps * 1e3
                es = 2 if dtype == "bf16" else 4
                nb = decode_mode_bytes(S, H, N, P, R, es, trap, rot)
                rows.append({"variant": name, "N": N, "dtype": dtype, "R": R,
                             "us_cold": cold, "us_back_to_back": b2b,
                             "hbm_gbs_cold": nb / (cold * 1e-6) / 1e9,
                             "hbm_frac_cold": nb / (cold * 1e-6) / 1e9 / HBM_PEAK_GBS,
                             "algorithmic_bytes": nb})
                del g, h, y
                torch.cuda.empty_cache()
    del scratch
    return rows


def probe_lib():
    """The copy kernels of libm3probe (bandwidth anchors; not the library)."""
    import ctypes
    probe = ctypes.CDLL(os.path.join(ROOT, "state_space_sequence_exp_amd", "libm3probe.so"))
    probe.m3probe_copy.restype = ctypes.c_int
    probe.m3probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int, ctypes.c_void_p]
    return probe


def equal_copy_us(nbytes, steps, scratch):
    """Cold per-call time (MALL evicted first, as for the kernels it is set
    beside) of the fastest probe copy that moves nbytes in all: half read,
    half written.  A kernel's time over this is its fraction of what a plain
    copy of the same traffic reaches, fixed launch and ramp costs included."""
    import numpy as np
    import torch
    probe = probe_lib()
    half = (nbytes // 2) // 16 * 16
    src = torch.empty(half // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    best = None
    for v in range(probe.m3probe_copy_variants()):
        def run():
            rc = probe.m3probe_copy(src.data_ptr(), dst.data_ptr(), half, v,
                                    torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError("copy probe variant %d failed: %d" % (v, rc))
        run()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for s0, e0 in evs:
            flush_mall(scratch)
            s0.record()
            run()
            e0.record()
        torch.cuda.synchronize()
        us = float(np.median([s0.elapsed_time(e0) for s0, e0 in evs])) * 1e3
        best = us if best is None else min(best, us)
    del src, dst
    return best


def block_passes(steps, log):
    """Block-side passes at the prefill bench shapes (batch 4, 16 heads,
    N = P = 64, bf16; T 2048 with R = 1 and T 4096 with R = 4): per-call
    time (last-level cache evicted before each call) and HBM bandwidth of
    the algorithmic bytes -- every input read once, every output written once,
    weights included."""
    import numpy as np
    import torch
    import state_space_sequence_exp_amd as m3
    from state_space_sequence_exp_amd import inputs as I
    scratch = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda:0")
    out = {}
    for T, R in ((2048, 1), (4096, 4)):
        nb, H, N, P, es = 4, 16, 64, 64, 2
        inp = I.block_inputs(nb, T, H, N, P, R, "bf16", seed=140 + R)
        g = upload(dict(x_raw=inp["x_raw"], B_raw=inp["B_raw"], C_raw=inp["C_raw"],
                        dtype="bf16"))
        w = {k: torch.from_numpy(inp[k]).to("cuda:0")
             for k in ("norm_B", "norm_C", "bias_B", "bias_C", "up", "down")}
        del inp
        X = torch.empty((nb, T, H, R, P), dtype=torch.bfloat16, device="cuda:0")
        Bo, Co = torch.empty_like(g["B"]), torch.empty_like(g["C"])
        yo = torch.empty((nb, T, H, P), dtype=torch.bfloat16, device="cuda:0")

        def pre():
            m3.block_prepass(g["x"], g["B"], g["C"], w["norm_B"], w["norm_C"], w["bias_B"],
                             w["bias_C"], w["up"], 1e-6, x_out=X, B_out=Bo, C_out=Co)

        def post():
            m3.block_postpass(X, w["down"], y_out=yo)

        rows = nb * T * H
        weights = (2 * H * N + 2 * H * R * N + H * R * P) * 4
        nbytes = {"prepass": rows * (P + 4 * R * N + R * P) * es + weights,
                  "postpass": rows * (R * P + P) * es + H * R * P * 4}
        for name, fn in (("prepass", pre), ("postpass", post)):
            fn()
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(steps)]
            for s0, e0 in evs:
                flush_mall(scratch)
                s0.record()
                fn()
                e0.record()
            torch.cuda.synchronize()
            us = float(np.median([s0.elapsed_time(e0) for s0, e0 in evs])) * 1e3
            gbs = nbytes[name] / (us * 1e-6) / 1e9
            cus = equal_copy_us(nbytes[name], steps, scratch)
            out["%s_b4_t%d_h16_n64_p64_r%d" % (name, T, R)] = {
                "us": us, "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                "algorithmic_bytes": nbytes[name],
                "equal_copy_us": cus, "frac_of_equal_copy": cus / us}
            log("block %s T=%d R=%d: %.1f us, %.0f GB/s (a copy of the same bytes: %.1f us)"
                % (name, T, R, us, gbs, cus))
        del g, w, X, Bo, Co, yo
        torch.cuda.empty_cache()
    del scratch
    return out


def backward_bench(steps, log):
    """m3_backward at the SISO prefill bench shape (batch 4, T 2048, 16 heads,
    N = P = 64, bf16 inputs, float32 gradients): cold per-call time (MALL
    flushed before each call).  Algorithmic bytes: every input and dy read
    once, every gradient written once; the implementation's own state
    traffic (at this shape the chunked path's N x P float states per 64-token
    chunk and head: the local state S_c written, read and rewritten as the
    entry state G_c by the chain, read twice by the gradient pass (as G_c
    and as G_{c+1}); the local adjoint D_c written, read and rewritten as
    dG_{c+1}, read once) is reported separately."""
    import numpy as np
    import torch
    import state_space_sequence_exp_amd as m3
    from state_space_sequence_exp_amd import inputs as I
    cfg = I.WORKLOADS[1]
    inp = I.config_inputs(1)
    g = upload(inp)
    del inp
    dy = torch.randn(g["x"].shape, device="cuda:0").to(g["x"].dtype)
    ws = torch.empty(m3.backward_workspace_size(cfg.batch, cfg.seqlen, cfg.nheads, cfg.P, cfg.N,
                                                cfg.R, g["x"].dtype),
                     dtype=torch.uint8, device="cuda:0")
    scratch = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda:0")

    def call():
        return m3.backward(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"], dy,
                           workspace=ws)
    call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for s0, e0 in evs:
        flush_mall(scratch)
        s0.record()
        call()
        e0.record()
    torch.cuda.synchronize()
    ms = float(np.median([s0.elapsed_time(e0) for s0, e0 in evs]))
    th = cfg.batch * cfg.seqlen * cfg.nheads
    es, R, N, P = 2, cfg.R, cfg.N, cfg.P
    nbytes = (th * (2 * R * P * es + 2 * R * N * es + 8 + (N // 2) * 4)      # x, dy, B, C, dt, lam, theta
              + th * (R * P * 4 + 2 * R * N * 4 + 8 + (N // 2) * 4)        # dx, dB, dC, ddt, dlam, dtheta
              + cfg.nheads * 8)                                            # A, dA
    nchunk = cfg.batch * cfg.nheads * ((cfg.seqlen + 63) // 64)
    state_bytes = nchunk * N * P * 4 * (5 + 4)   # S/G: 1 + 2 + 2 accesses, D/dG: 1 + 2 + 1
    gbs = nbytes / (ms * 1e-3) / 1e9
    log("backward: %.3f ms, %.0f GB/s algorithmic" % (ms, gbs))
    del g, dy, ws, scratch
    torch.cuda.empty_cache()
    return {"ms": ms, "tokens_per_s": cfg.batch * cfg.seqlen / (ms * 1e-3), "hbm_gbs": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
            "checkpoint_bytes": state_bytes,
            "state_traffic_gbs": state_bytes / (ms * 1e-3) / 1e9}


def upload(inp):
    import numpy as np
    import torch
    dev = torch.device("cuda:0")

    def st(raw):
        if inp["dtype"] == "bf16":
            return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32)).to(dev)

    g = {k: st(inp[k + "_raw"]) for k in ("x", "B", "C")}
    for k in ("dt", "lam", "theta", "A"):
        if k in inp:
            g[k] = torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.float32)).to(dev)
    if "h0" in inp:
        g["h0"] = torch.from_numpy(np.ascontiguousarray(inp["h0"], dtype=np.float32)).to(dev)
    return g


def time_prefill(cfg, g, steps, warmup, flush=True):
    """Per-call durations (ms) of m3_prefill with HIP events on the current
    stream; a MALL flush (flush_mall) before each call."""
    import torch
    import state_space_sequence_exp_amd as m3
    dev = torch.device("cuda:0")
    ws_bytes = m3.prefill_workspace_size(cfg.batch, cfg.seqlen, cfg.nheads, cfg.P, cfg.N, cfg.R,
                                         cfg.chunk, g["x"].dtype)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    y = torch.empty_like(g["x"])
    hf = torch.empty((cfg.batch, cfg.nheads, cfg.N, cfg.P), dtype=torch.float32, device=dev)
    scratch = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev) if flush else None

    def call():
        m3.prefill(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"], cfg.chunk,
                   y=y, h_final=hf, workspace=ws)

    # warm-up takes the timed sequence itself (flush, then the call), so the
    # first touch of the scratch buffer and of the events is not timed
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(max(steps, warmup))]
    for s, e in evs[:warmup]:
        if flush:
            flush_mall(scratch)
        s.record()
        call()
        e.record()
    torch.cuda.synchronize()
    evs = evs[:steps]
    for s, e in evs:
        if flush:
            flush_mall(scratch)
        s.record()
        call()
        e.record()
    torch.cuda.synchronize()
    times = [s.elapsed_time(e) for s, e in evs]
    # back-to-back (no flush) for reference
    s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(steps):
        call()
    e0.record()
    torch.cuda.synchronize()
    b2b = s0.elapsed_time(e0) / steps
    if ws_bytes > 0:
        err = m3.prefill_workspace_error(ws)
        if err != 0:
            raise RuntimeError("prefill chain error word %d after the timed calls of %s "
                               "(a timed-out wait or dirty counters): outputs invalid"
                               % (err, cfg.name))
    del scratch
    return times, b2b


def time_decode(cfg, g, steps, warmup, matrix_cores=False):
    import torch
    import state_space_sequence_exp_amd as m3
    K = g["x"].shape[0]
    h = g["h0"].clone()
    y = torch.empty((cfg.batch, cfg.nheads, cfg.R, cfg.P), dtype=g["x"].dtype, device=h.device)

    def step(t):
        cur, prev = t % K, (t - 1) % K
        m3.decode_step(h, g["x"][cur], g["x"][prev], g["B"][cur], g["B"][prev], g["C"][cur],
                       g["dt"][cur], g["A"], g["lam"][cur], g["theta"][cur], y=y,
                       matrix_cores=matrix_cores)

    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    reps = []
    for _ in range(3):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for t in range(steps):
            step(t)
        e.record()
        torch.cuda.synchronize()
        reps.append(s.elapsed_time(e) / steps)
    reps.sort()
    return reps[len(reps) // 2]


def host_cpu():
    """(cores this process may run on, cores the oracle uses, CPU model)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    # one GPU's share of the host: at most 16 worker threads
    return avail, max(1, min(avail, 16)), model


def cpu_baseline(cfg, inp, budget_s=20.0):
    """The fp64 oracle on the host cores: whole (b, h) units of the same
    workload, as many as fit the time budget; scaled to tokens/s of the full
    workload (units are independent)."""
    import oracle
    avail, cores, model = host_cpu()
    nunits = cfg.batch * cfg.nheads
    # calibrate with one wave of `cores` units, then run a sample within budget
    n = min(nunits, cores)
    t0 = time.perf_counter()
    oracle.prefill(inp["x"], inp["dt"], inp["A"], inp["lam"], inp["theta"], inp["B"], inp["C"],
                   units=list(range(n)), nthreads=cores)
    dt = time.perf_counter() - t0
    waves = max(1, min(nunits // cores, int(budget_s / max(dt, 1e-6))))
    n2 = min(nunits, waves * cores)
    if n2 > n:
        t0 = time.perf_counter()
        oracle.prefill(inp["x"], inp["dt"], inp["A"], inp["lam"], inp["theta"], inp["B"],
                       inp["C"], units=list(range(n2)), nthreads=cores)
        dt = time.perf_counter() - t0
        n = n2
    # the whole workload fits the budget: repeat it so the time is not a
    # single short measurement
    reps = 1
    if n == nunits and dt < budget_s / 2:
        reps = max(1, min(100, int(budget_s / 2 / max(dt, 1e-6))))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.prefill(inp["x"], inp["dt"], inp["A"], inp["lam"], inp["theta"], inp["B"],
                           inp["C"], units=list(range(n)), nthreads=cores)
        dt = (time.perf_counter() - t0) / reps
    full_time = dt * nunits / n
    return {"value": cfg.batch * cfg.seqlen / full_time, "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cores_available": avail, "cores_capped_at": 16,
            "cpu_model": model,
            "sample": "%d of %d (batch, head) units over all %d tokens, fp64 C oracle, "
                      "%d run(s) of %.3g s" % (n, nunits, cfg.seqlen, reps, dt)}


def cpu_baseline_decode(cfg, inp, steps=10):
    """The fp64 oracle's decode step on the full batch (every sequence and
    head), timed over `steps` consecutive steps: us per step."""
    import numpy as np
    import oracle
    avail, cores, model = host_cpu()
    K = inp["x"].shape[0]
    h = inp["h0"].astype(np.float64)
    t0 = time.perf_counter()
    for t in range(steps):
        cur, prev = t % K, (t - 1) % K
        _, h = oracle.decode_step(h, inp["x"][cur], inp["x"][prev], inp["B"][cur],
                                  inp["B"][prev], inp["C"][cur], inp["dt"][cur], inp["A"],
                                  inp["lam"][cur], inp["theta"][cur], nthreads=cores)
    us = (time.perf_counter() - t0) / steps * 1e6
    return {"value": us, "unit": "us/step", "cores": cores, "kind": "oracle",
            "cores_available": avail, "cores_capped_at": 16, "cpu_model": model,
            "sample": "full batch (%d sequences x %d heads), %d consecutive steps"
                      % (cfg.batch, cfg.nheads, steps)}


def device_anchors(log):
    """Measured peaks of this GPU, beside the published ones: a 512 MiB
    device-to-device copy (read + write, GB/s) and a large bf16 GEMM
    (TFLOP/s), each the median of several event-timed repeats."""
    import numpy as np
    import torch
    n = 512 * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    probe = probe_lib()

    def probe_copy(variant):
        def run():
            rc = probe.m3probe_copy(src.data_ptr(), dst.data_ptr(), n * 4, variant,
                                    torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError("copy probe variant %d failed: %d" % (variant, rc))
        return run

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(10):
            s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record()
            fn()
            e0.record()
            torch.cuda.synchronize()
            ts.append(s0.elapsed_time(e0))
        return float(np.median(ts))

    # the anchor is the fastest of the probe's plain copy variants
    per_variant = []
    for v in range(probe.m3probe_copy_variants()):
        dst.zero_()
        per_variant.append(timed(probe_copy(v)))
        if not torch.equal(dst[-(1 << 20):], src[-(1 << 20):]):
            raise RuntimeError("copy probe variant %d produced wrong data" % v)
    best = int(np.argmin(per_variant))
    ms = per_variant[best]
    copy_gbs = 2 * n * 4 / (ms * 1e-3) / 1e9
    tms = timed(lambda: dst.copy_(src))
    torch_gbs = 2 * n * 4 / (tms * 1e-3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn(m, m, device="cuda:0").to(torch.bfloat16)
    b = torch.randn(m, m, device="cuda:0").to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    ts = []
    for _ in range(10):
        s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        torch.matmul(a, b)
        e0.record()
        torch.cuda.synchronize()
        ts.append(s0.elapsed_time(e0))
    gms = float(np.median(ts))
    tflops = 2 * m ** 3 / (gms * 1e-3) / 1e12
    del a, b
    torch.cuda.empty_cache()
    log("anchors: copy %.0f GB/s (torch copy_ %.0f), bf16 GEMM %.0f TFLOP/s"
        % (copy_gbs, torch_gbs, tflops))
    return {"hbm_copy_gbs": copy_gbs,
            "hbm_copy": "512 MiB device-to-device copy (read + write) by the fastest of %d "
                        "streaming HIP copy kernels (libm3probe: 16-byte vectors, 4/8/16 per "
                        "thread, ordinary or non-temporal), variant %d, median of 10, %.3f ms"
                        % (len(per_variant), best, ms),
            "hbm_copy_variants_gbs": [2 * n * 4 / (t * 1e-3) / 1e9 for t in per_variant],
            "torch_copy_gbs": torch_gbs,
            "bf16_gemm_tflops": tflops,
            "bf16_gemm": "torch.matmul bf16 %dx%dx%d, median of 10, %.3f ms" % (m, m, m, gms),
            "hbm_peak_spec_gbs": HBM_PEAK_GBS, "bf16_peak_spec_tflops": BF16_PEAK_TFLOPS}


def counter_sequence():
    """Fixed, untimed workload for hardware-counter runs (see --counters)."""
    import torch
    import state_space_sequence_exp_amd as m3
    from state_space_sequence_exp_amd import inputs as I
    for idx, reps in ((1, 3), (3, 1), (2, 1)):
        cfg = I.WORKLOADS[idx]
        g = upload(I.config_inputs(idx))
        for _ in range(reps):
            m3.prefill(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"], cfg.chunk)
        torch.cuda.synchronize()
        del g
    c = I.WORKLOADS[4]
    g = upload(I.decode_config_inputs(ring=2))
    h = g["h0"].clone()
    for t in range(10):
        cur, prev = t % 2, (t + 1) % 2
        m3.decode_step(h, g["x"][cur], g["x"][prev], g["B"][cur], g["B"][prev], g["C"][cur],
                       g["dt"][cur], g["A"], g["lam"][cur], g["theta"][cur])
    torch.cuda.synchronize()
    del g, h
    # the backward at the SISO shape, then the MIMO block passes (B4 T4096 H16
    # N = P = 64, R = 4), once each
    cfg = I.WORKLOADS[1]
    g = upload(I.config_inputs(1))
    dy = torch.randn(g["x"].shape, device="cuda:0").to(g["x"].dtype)
    m3.backward(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"], dy)
    torch.cuda.synchronize()
    del g, dy
    nb, T, H, N, P, R = 4, 4096, 16, 64, 64, 4
    inp = I.block_inputs(nb, T, H, N, P, R, "bf16", seed=144)
    g = upload(dict(x_raw=inp["x_raw"], B_raw=inp["B_raw"], C_raw=inp["C_raw"], dtype="bf16"))
    w = {k: torch.from_numpy(inp[k]).to("cuda:0")
         for k in ("norm_B", "norm_C", "bias_B", "bias_C", "up", "down")}
    X, _, _ = m3.block_prepass(g["x"], g["B"], g["C"], w["norm_B"], w["norm_C"], w["bias_B"],
                               w["bias_C"], w["up"], 1e-6)
    m3.block_postpass(X, w["down"])
    torch.cuda.synchronize()
    del g, w, X, inp
    src = torch.ones(128 * 1024 * 1024, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("counter sequence done (copy of %d bytes)" % (src.numel() * 4))


# ---------------------------------------------------------------------------
# The goals set for these kernels: prefill at half the dense bf16 MFMA peak,
# the decode step at 70% of the HBM peak.
PREFILL_MFMA_GOAL = 0.5
DECODE_HBM_GOAL = 0.7


def goals_report(line):
    """Each goal beside what was measured.  For prefill also the MFMA
    fraction its useful flops would reach if the call ran at the HBM
    roofline (its algorithmic bytes at 8 TB/s): the most the shape allows
    while it stays bound by its bytes."""
    from state_space_sequence_exp_amd import inputs as I

    def ceiling(c):
        t_s = prefill_bytes(c) / (HBM_PEAK_GBS * 1e9)
        return prefill_flops(c) / t_s / 1e12 / BF16_PEAK_TFLOPS

    pre = {"goal": PREFILL_MFMA_GOAL, "measured": {}, "ceiling_at_hbm_roofline": {}}
    c1 = I.WORKLOADS[1]
    pre["measured"][c1.name] = line["roofline"]["mfma_frac"]
    pre["ceiling_at_hbm_roofline"][c1.name] = ceiling(c1)
    sec = line.get("secondary", {})
    for idx in (2, 3):
        c = I.WORKLOADS[idx]
        if c.name in sec:
            pre["measured"][c.name] = sec[c.name]["mfma_frac"]
            pre["ceiling_at_hbm_roofline"][c.name] = ceiling(c)
    out = {"prefill_bf16_mfma_frac": pre}
    c4 = I.WORKLOADS[4]
    if c4.name in sec:
        out["decode_hbm_frac"] = {"goal": DECODE_HBM_GOAL,
                                  "measured": sec[c4.name]["roofline"]["frac"]}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-flush", action="store_true", help="do not evict the MALL between steps")
    ap.add_argument("--no-decode-sweep", action="store_true")
    ap.add_argument("--no-block", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="short untimed sequence for rocprofv3 counter runs: SISO prefill x3, "
                         "long SISO prefill x1, MIMO prefill x1, 10 decode steps, the SISO "
                         "backward x1, the MIMO block passes x1, and a 512 MiB device copy x3 "
                         "(the copy calibrates the byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (every "
              "(batch, head) unit is independent, so a batch or its heads split across GPUs "
              "with no communication)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import state_space_sequence_exp_amd as m3
    from state_space_sequence_exp_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    m3.load_library()
    if args.counters:
        counter_sequence()
        return

    # measured peaks of this GPU (context for every fraction below)
    anchors = device_anchors(log)
    copy_gbs = anchors["hbm_copy_gbs"]

    # ---- headline: SISO prefill (configuration 1) ----
    cfg = I.WORKLOADS[1]
    log("generating %s" % cfg.name)
    inp = I.config_inputs(1)
    g = upload(inp)
    log("timing prefill %s: %d warmup + %d steps" % (cfg.name, args.warmup, args.steps))
    times, b2b = time_prefill(cfg, g, args.steps, args.warmup, flush=not args.no_flush)
    ms = float(np.mean(times))
    if max(times) > 3 * float(np.median(times)):
        log("note: slowest timed step %.3f ms against a median of %.3f ms"
            % (max(times), float(np.median(times))))
    tokens = cfg.batch * cfg.seqlen
    value = tokens / (ms * 1e-3)
    nbytes = prefill_bytes(cfg)
    achieved = nbytes / (ms * 1e-3) / 1e9
    traffic = measured_traffic("prefill_config1")
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": float(np.median(times)),
        "ms_each_step": [round(t, 4) for t in times],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "SISO prefill: batch 4, T=2048, 16 heads, N=64, P=64, R=1, "
                               "bf16 x/B/C, fp32 state, chunk 64",
                   "global_batch": cfg.batch, "seq_len": cfg.seqlen, "parallelism": "none"},
        "roofline": {"kernel": "prefill_tok1_kernel (single-pass token-lane fused chained prefill, one launch per m3_prefill call)",
                     "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": nbytes,
                     "frac_of_measured_copy": achieved / copy_gbs,
                     "mfma_frac": prefill_flops(cfg) / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "prefill_ms_back_to_back_no_flush": b2b,
        "device_anchors": anchors,
    }

    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        line["cpu_baseline"] = cpu_baseline(cfg, inp)
    del g, inp
    torch.cuda.empty_cache()

    if not args.no_secondary:
        sec = {}
        # configuration 0: latency only (a few hundred tokens: launch-bound)
        c = I.WORKLOADS[0]
        ii = I.config_inputs(0)
        gg = upload(ii)
        log("timing prefill %s" % c.name)
        tt, bb = time_prefill(c, gg, args.steps, args.warmup, flush=not args.no_flush)
        sec[c.name] = {"us": float(np.median(tt)) * 1e3, "us_back_to_back_no_flush": bb * 1e3,
                       "tokens_per_s": c.batch * c.seqlen / (float(np.median(tt)) * 1e-3)}
        if not args.no_cpu_baseline:
            sec[c.name]["cpu_baseline"] = cpu_baseline(c, ii, budget_s=2.0)
        del gg, ii
        for idx in (2, 3):
            c = I.WORKLOADS[idx]
            log("generating %s" % c.name)
            ii = I.config_inputs(idx)
            gg = upload(ii)
            steps = max(3, args.steps // 2)
            log("timing prefill %s" % c.name)
            tt, bb = time_prefill(c, gg, steps, max(1, args.warmup // 2), flush=not args.no_flush)
            m = float(np.mean(tt))
            nb = prefill_bytes(c)
            sec[c.name] = {"tokens_per_s": c.batch * c.seqlen / (m * 1e-3), "ms": m,
                           "ms_back_to_back_no_flush": bb, "hbm_gbs": nb / (m * 1e-3) / 1e9,
                           "hbm_frac": nb / (m * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "hbm_frac_of_measured_copy": nb / (m * 1e-3) / 1e9 / copy_gbs,
                           "mfma_frac": prefill_flops(c) / (m * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                           "algorithmic_bytes": nb, "chunk": c.chunk}
            del gg
            torch.cuda.empty_cache()
            if not args.no_cpu_baseline:
                log("cpu baseline %s" % c.name)
                sec[c.name]["cpu_baseline"] = cpu_baseline(c, ii, budget_s=10.0)
            del ii
        c = I.WORKLOADS[4]
        log("generating %s" % c.name)
        ii = I.decode_config_inputs()
        gg = upload(ii)
        log("timing decode: %d steps x 3" % args.decode_steps)
        us = time_decode(c, gg, args.decode_steps, 10) * 1e3
        nb = decode_bytes(c)
        gbs = nb / (us * 1e-6) / 1e9
        sec[c.name] = {"us_per_step": us, "hbm_gbs": gbs,
                       "roofline": {"kernel": "decode_kernel", "bound": "hbm", "achieved": gbs,
                                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                    "frac": gbs / HBM_PEAK_GBS,
                                    "traffic": measured_traffic("decode_config4"),
                                    "algorithmic_bytes": nb,
                                    "frac_of_measured_copy": gbs / copy_gbs}}
        # the same steps with the rank-2R update on the matrix cores
        log("timing decode (matrix-core variant): %d steps x 3" % args.decode_steps)
        us_m = time_decode(c, gg, args.decode_steps, 10, matrix_cores=True) * 1e3
        gbs_m = nb / (us_m * 1e-6) / 1e9
        sec[c.name]["mfma_variant"] = {"kernel": "decode_mfma_kernel (m3_decode_step_mfma)",
                                       "us_per_step": us_m, "hbm_gbs": gbs_m,
                                       "frac": gbs_m / HBM_PEAK_GBS,
                                       "frac_of_measured_copy": gbs_m / copy_gbs}
        del gg
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            log("cpu baseline decode")
            sec[c.name]["cpu_baseline"] = cpu_baseline_decode(c, ii, steps=10)
        del ii
        if not args.no_decode_sweep:
            sec["decode_sweep_b128_h64_p64"] = decode_sweep(20, log)
        if not args.no_block:
            sec["block_passes"] = block_passes(20, log)
        if not args.no_backward:
            sec["backward_siso_b4_t2048_h16_n64_p64"] = backward_bench(10, log)
        line["secondary"] = sec
    line["goals"] = goals_report(line)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
