"""Build libm3ssm.so (HIP for gfx950) in-tree.

    python -m state_space_sequence_exp_amd.build

compiles every ``csrc/*.hip`` with hipcc for gfx950 (in parallel) and links
``state_space_sequence_exp_amd/libm3ssm.so``.  Packed-fp32 VALU instructions
are disabled for all device code.
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


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = _hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources under " + CSRC)
    tmp = tempfile.mkdtemp(prefix="m3ssm_build_")
    try:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [hipcc] + compile_flags() + ["-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
            if verbose:
                sys.stderr.write(r.stderr)
            return obj

        with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
            objs = list(ex.map(compile_one, srcs))
        out_tmp = LIB_PATH + ".tmp%d" % os.getpid()
        cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", out_tmp] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
        os.replace(out_tmp, LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
