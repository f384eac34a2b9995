"""Host sanitizer runs (CPU only): the fp64 oracle and the host side of
libm3ssm (argument validation, workspace carving, shape rules) built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven by the small C
programs under tests/sanitize/.  Only host code is instrumented (every
sanitizer flag of a HIP compile sits behind -Xarch_host); the drivers make
no GPU call.  The sanitized library is cached under _build/sanitize/, keyed
by a hash of the sources and flags."""
import hashlib
import glob
import os
import subprocess

import pytest

from state_space_sequence_exp_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
DRIVERS = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n--- stdout\n%s\n--- stderr\n%s" % (" ".join(cmd), r.stdout,
                                                                     r.stderr[-6000:])
    return r


def _sources_hash():
    h = hashlib.sha256(" ".join(B.compile_flags() + HOST_SAN).encode())
    srcs = [f for f in glob.glob(os.path.join(B.CSRC, "*")) if os.path.isfile(f)]
    for f in sorted(srcs) + [os.path.join(B.INCLUDE, "m3ssm.h")]:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


@pytest.fixture(scope="module")
def sanitized_library():
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "libm3ssm_san_%s.so" % _sources_hash())
    if not os.path.exists(lib):
        for old in glob.glob(os.path.join(OUT, "libm3ssm_san_*.so")):
            os.remove(old)
        B.build(extra_flags=HOST_SAN, out=lib)
    return lib


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "driver_oracle")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-pthread",
          os.path.join(DRIVERS, "driver_oracle.c"), os.path.join(ROOT, "oracle", "m3_oracle.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert "0 failures" in r.stdout
    assert "runtime error" not in r.stderr


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not found")
def test_host_validation_under_asan_ubsan(sanitized_library, tmp_path):
    exe = str(tmp_path / "driver_abi")
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-I", B.INCLUDE, os.path.join(DRIVERS, "driver_abi.c"),
          sanitized_library, "-Wl,-rpath," + os.path.dirname(sanitized_library), "-o", exe])
    r = _run([exe], env=ENV)
    assert " 0 failures" in r.stdout
    assert "runtime error" not in r.stderr
