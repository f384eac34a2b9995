"""Build libm3ssm.so (HIP for gfx950) in-tree.

    python -m state_space_sequence_exp_amd.build

compiles every ``csrc/*.hip`` with hipcc for gfx950 (in parallel) and links
``state_space_sequence_exp_amd/libm3ssm.so``.  Packed-fp32 VALU instructions
are disabled for all device code; a few prefill sources take a measured
instruction-scheduling strategy (SCHED).
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libm3ssm.so")
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libm3ssm")


def compile_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


# Instruction-scheduling strategy per source file, where a measured one beats
# the default: the kernels are latency-bound at few waves per SIMD, and
# LLVM's AMDGPU schedulers trade registers for latency hiding differently
# per shape.  Cold per-call times against the default on one MI355X:
# - N = 128 SISO prefill (B1 T16384 H64 P64): 559 -> 515 us, iterative-ilp;
# - MIMO R = 4 prefill (B4 T4096 H16 N64 P64): 278 -> 274 us, iterative-ilp;
# - N = 64 SISO prefill (B4 T2048 H16 P64): 67.7 -> 66.2 us,
#   max-memory-clause (iterative-ilp: 67.8);
# - decode, S256 H32 N128 P64 R4 bf16: 89.9 -> 87.6 us, and S128 H64 N64
#   R4 fp32: 57.1 -> 51.0 us, iterative-ilp;
# - backward, SISO B4 T2048 H16 N64 P64: 1.061 -> 1.044 ms,
#   max-memory-clause.
SCHED = {
    "prefill_bf16_r1.hip": "max-memory-clause",
    "prefill_bf16_r1_n128.hip": "iterative-ilp",
    "prefill_bf16_r4.hip": "iterative-ilp",
    "decode.hip": "iterative-ilp",
    "backward.hip": "max-memory-clause",
}


def file_flags(src: str):
    st = SCHED.get(os.path.basename(src))
    return ["-mllvm", "-amdgpu-sched-strategy=" + st] if st else []


def build(verbose: bool = False, jobs: int = 8, extra_flags=(), out: str = LIB_PATH) -> str:
    """Compile every source and link the shared library at `out` (default:
    the in-tree libm3ssm.so).  extra_flags go to every compile line (for
    instance host-only sanitizer flags, each behind -Xarch_host)."""
    hipcc = _hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources under " + CSRC)
    tmp = tempfile.mkdtemp(prefix="m3ssm_build_")
    try:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = ([hipcc] + compile_flags() + file_flags(src) + list(extra_flags)
                   + ["-c", src, "-o", obj])
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
            if verbose:
                sys.stderr.write(r.stderr)
            return obj

        with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
            objs = list(ex.map(compile_one, srcs))
        out_tmp = out + ".tmp%d" % os.getpid()
        cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", out_tmp] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
        os.replace(out_tmp, out)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out


PROBE_SRC = os.path.join(CSRC, "probe", "copy_probe.hip")
PROBE_PATH = os.path.join(PKG, "libm3probe.so")


def build_probe() -> str:
    """The copy kernel that anchors bandwidth measurements (libm3probe.so)."""
    out_tmp = PROBE_PATH + ".tmp%d" % os.getpid()
    cmd = [_hipcc()] + compile_flags() + ["-shared", PROBE_SRC, "-o", out_tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (PROBE_SRC, r.stdout, r.stderr))
    os.replace(out_tmp, PROBE_PATH)
    return PROBE_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe())
