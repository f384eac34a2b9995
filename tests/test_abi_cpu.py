"""CPU-only checks of the C ABI: the library loads, exports every function
include/m3ssm.h declares, and rejects invalid calls on the host before any
HIP call (so no GPU is needed for these paths)."""
import ctypes
import os
import re

import pytest

import state_space_sequence_exp_amd as m3
from state_space_sequence_exp_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "m3ssm.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(m3.LIB_PATH):
        from state_space_sequence_exp_amd import build
        build.build()
    return m3.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(m3_[a-z_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(_binding.ABI_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.m3_version() == 150
    for code in range(6):
        s = m3.status_string(code)
        assert s.startswith("M3_")
    assert "unknown" in m3.status_string(99)


def test_workspace_error_validation(lib):
    """Invalid workspaces are rejected on the host, before any HIP call."""
    word = ctypes.c_int(-7)
    f = lib.m3_prefill_workspace_error
    assert f(None, 4096, 0, ctypes.byref(word), None) == m3.M3_ERR_INVALID_VALUE
    buf = ctypes.create_string_buffer(4096 + 512)
    base = ctypes.addressof(buf)
    aligned = (base + 255) // 256 * 256
    assert f(ctypes.c_void_p(aligned + 4), 4096, 0, ctypes.byref(word), None) == \
        m3.M3_ERR_INVALID_VALUE
    assert f(ctypes.c_void_p(aligned), 8, 0, ctypes.byref(word), None) == m3.M3_ERR_INVALID_VALUE
    assert word.value == -7


def dims(b=1, t=64, h=1, p=16, n=16, r=1):
    return _binding.M3Dims(b, t, h, p, n, r)


def ws(d, chunk=32, dtype=m3.M3_F32):
    return _binding.load_library().m3_prefill_workspace_size(ctypes.byref(d), chunk, dtype)


def test_workspace_size(lib):
    """The chain counters (256 words: the ticket counters, the error word,
    the finished-workgroup count; then one status word per workgroup), from
    8 KiB or past the counters one slot per workgroup (two states, the
    rotation per pair, the decay and three unused floats), then one
    continuation entry state per (batch, head) unit."""
    r256 = lambda v: (v + 255) // 256 * 256

    def expect(nb, nt, nh, p, n, chunk):
        units = nb * nh
        nc = max(1, -(-nt // chunk))
        k = min(nc, max(1, -(-(nc * units) // 256)))
        grid = units * (-(-nc // k))
        slots = max(8192, r256((256 + grid) * 4))
        return r256(slots + r256(grid * (2 * n * p + n + 4) * 4) + units * n * p * 4)

    d = dims(2, 100, 3, 16, 32, 2)     # 6 units, 4 chunks of 32: 24 segments
    assert ws(d, 32, m3.M3_F32) == expect(2, 100, 3, 16, 32, 32)
    assert ws(d, 32, m3.M3_BF16) == expect(2, 100, 3, 16, 32, 32)
    # 8 KiB of counters, 24 slots of 1060 floats (101888 bytes), 6 entry states
    assert expect(2, 100, 3, 16, 32, 32) == 8192 + 101888 + 6 * 512 * 4
    d = dims(64, 100, 40, 16, 32, 1)   # 2560 units, one segment each: counters past 8 KiB
    assert ws(d, 32, m3.M3_BF16) == expect(64, 100, 40, 16, 32, 32)
    assert expect(64, 100, 40, 16, 32, 32) == r256(2816 * 4) + r256(2560 * 1060 * 4) + 2560 * 2048
    assert ws(dims(0, 100), 32) == 0
    assert ws(dims(1, 0), 32) == 0


@pytest.mark.parametrize("bad,code", [
    (dict(n=15), m3.M3_ERR_INVALID_VALUE),      # odd N
    (dict(r=0), m3.M3_ERR_INVALID_VALUE),       # R < 1
    (dict(h=0), m3.M3_ERR_INVALID_VALUE),       # no heads
    (dict(t=-1), m3.M3_ERR_INVALID_VALUE),
    (dict(p=24), m3.M3_ERR_NOT_SUPPORTED),      # P outside {16,32,64,128}
    (dict(r=3), m3.M3_ERR_NOT_SUPPORTED),
    (dict(n=18), m3.M3_ERR_NOT_SUPPORTED),      # N not a multiple of 16
    (dict(n=512), m3.M3_ERR_NOT_SUPPORTED),
])
def test_prefill_shape_validation(lib, bad, code):
    d = dims(**bad)
    fake = ctypes.c_void_p(0x10000)
    st = lib.m3_prefill(ctypes.byref(d), m3.M3_F32, 32, fake, fake, fake, fake, fake, fake, fake,
                        fake, None, fake, 1 << 30, None)
    assert st == code
    assert ws(d) == 0


def test_prefill_chunk_validation(lib):
    d = dims()
    fake = ctypes.c_void_p(0x10000)
    call = lambda chunk, dtype=m3.M3_F32, dd=d: lib.m3_prefill(
        ctypes.byref(dd), dtype, chunk, fake, fake, fake, fake, fake, fake, fake, fake, None,
        fake, 1 << 30, None)
    assert call(0) == m3.M3_ERR_INVALID_VALUE
    assert call(-16) == m3.M3_ERR_INVALID_VALUE
    assert call(24) == m3.M3_ERR_NOT_SUPPORTED       # not a multiple of 16
    assert call(256) == m3.M3_ERR_NOT_SUPPORTED      # above 128
    assert call(128, dd=dims(r=4)) == m3.M3_ERR_NOT_SUPPORTED   # chunk * R > 256
    assert call(32, dtype=7) == m3.M3_ERR_INVALID_VALUE
    assert call(32, dtype=m3.M3_BF16) == m3.M3_ERR_NOT_SUPPORTED  # bf16 needs N % 32 == 0


def test_prefill_pointer_and_workspace_validation(lib):
    d = dims()
    ok = ctypes.c_void_p(0x10000)
    mis = ctypes.c_void_p(0x10001)
    need = ws(d)
    assert need > 0
    args = [ok] * 8
    base = lambda a, h=None, w=ok, wb=need: lib.m3_prefill(
        ctypes.byref(d), m3.M3_F32, 32, *a, h, w, wb, None)
    for i in range(8):  # each input / output pointer null or misaligned
        a = list(args)
        if i not in (3, 4):  # lam and theta are optional (the reduced forms)
            a[i] = None
            assert base(a) == m3.M3_ERR_INVALID_VALUE
        a[i] = mis
        assert base(a) == m3.M3_ERR_INVALID_VALUE
    # without lam and theta the remaining checks still apply
    a = list(args)
    a[3] = a[4] = None
    a[7] = mis
    assert base(a) == m3.M3_ERR_INVALID_VALUE
    assert base(args, h=mis) == m3.M3_ERR_INVALID_VALUE
    a = list(args)
    a[0] = ctypes.c_void_p(0x10004)   # x must be 16-byte aligned
    assert base(a) == m3.M3_ERR_INVALID_VALUE
    assert base(args, w=None) == m3.M3_ERR_WORKSPACE
    assert base(args, wb=need - 1) == m3.M3_ERR_WORKSPACE
    assert base(args, w=ctypes.c_void_p(0x10010)) == m3.M3_ERR_INVALID_VALUE  # not 256-aligned
    # nothing to do: succeeds without touching the device
    d0 = dims(b=0)
    assert lib.m3_prefill(ctypes.byref(d0), m3.M3_F32, 32, None, None, None, None, None, None,
                          None, None, None, None, 0, None) == m3.M3_SUCCESS
    assert lib.m3_prefill(None, m3.M3_F32, 32, *args, None, ok, need, None) == m3.M3_ERR_INVALID_VALUE


def test_prefill_from_state_validation(lib):
    """The continuation entry point validates like m3_prefill, plus its own
    pointers: x_prev and B_prev together, element alignment, and h_final equal
    to h0 or disjoint from it."""
    d = dims(b=2, h=3, p=16, n=32, r=2)
    ok = ctypes.c_void_p(0x100000)
    mis = ctypes.c_void_p(0x100001)
    need = ws(d)
    hbytes = 2 * 3 * 32 * 16 * 4
    args = [ok] * 8          # x, dt, A, lam, theta, B, C, y

    def call(h0=None, xp=None, bp=None, hf=None, dd=d, a=args, w=ok, wb=need):
        return lib.m3_prefill_from_state(ctypes.byref(dd), m3.M3_F32, 32, h0, xp, bp, *a, hf, w,
                                         wb, None)
    assert call(xp=ok) == m3.M3_ERR_INVALID_VALUE            # x_prev without B_prev
    assert call(bp=ok) == m3.M3_ERR_INVALID_VALUE            # B_prev without x_prev
    assert call(h0=mis) == m3.M3_ERR_INVALID_VALUE
    assert call(xp=mis, bp=ok) == m3.M3_ERR_INVALID_VALUE
    assert call(xp=ok, bp=mis) == m3.M3_ERR_INVALID_VALUE
    h0 = 0x200000
    # h_final partially overlapping h0
    assert call(h0=ctypes.c_void_p(h0), hf=ctypes.c_void_p(h0 + 256)) == m3.M3_ERR_INVALID_VALUE
    assert call(h0=ctypes.c_void_p(h0 + 256), hf=ctypes.c_void_p(h0)) == m3.M3_ERR_INVALID_VALUE
    # the shared checks still apply
    assert call(dd=dims(n=15)) == m3.M3_ERR_INVALID_VALUE
    assert call(h0=ok, w=None) == m3.M3_ERR_WORKSPACE
    bad = list(args)
    bad[0] = None
    assert call(h0=ok, a=bad) == m3.M3_ERR_INVALID_VALUE
    # nothing to do: succeeds without touching the device
    d0 = dims(b=0)
    assert lib.m3_prefill_from_state(ctypes.byref(d0), m3.M3_F32, 32, ok, ok, ok, None, None,
                                     None, None, None, None, None, None, None, None, 0,
                                     None) == m3.M3_SUCCESS
    # disjoint h_final, and h_final == h0, pass validation (checked here with a
    # null workspace, which is reported after the pointer checks)
    assert call(h0=ctypes.c_void_p(h0), hf=ctypes.c_void_p(h0 + hbytes),
                w=None) == m3.M3_ERR_WORKSPACE
    assert call(h0=ctypes.c_void_p(h0), hf=ctypes.c_void_p(h0), w=None) == m3.M3_ERR_WORKSPACE


def test_decode_validation(lib):
    fake = ctypes.c_void_p(0x10000)
    mis = ctypes.c_void_p(0x10001)

    def call(d, dtype=m3.M3_BF16, h_in=fake, h_out=fake, others=None):
        o = others or [fake] * 10
        return lib.m3_decode_step(ctypes.byref(d), dtype, h_in, h_out, *o, None)

    assert call(dims(b=2, n=15)) == m3.M3_ERR_INVALID_VALUE
    assert call(dims(b=2, r=3)) == m3.M3_ERR_NOT_SUPPORTED
    assert call(dims(b=2, p=128, n=256)) == m3.M3_ERR_NOT_SUPPORTED
    assert call(dims(b=2), dtype=5) == m3.M3_ERR_INVALID_VALUE
    assert call(dims(b=0)) == m3.M3_SUCCESS
    # others: x_t, x_prev, B_t, B_prev, C_t, dt, A, lam, theta, y_t
    for i in range(10):
        o = [fake] * 10
        if i not in (7, 8):  # lam and theta are optional
            o[i] = None
            assert call(dims(b=2), others=o) == m3.M3_ERR_INVALID_VALUE
        o[i] = mis
        assert call(dims(b=2), others=o) == m3.M3_ERR_INVALID_VALUE
    # without lam, x_prev and B_prev may be null; the other checks still apply
    o = [fake] * 10
    o[1] = o[3] = o[7] = None
    o[9] = mis
    assert call(dims(b=2), others=o) == m3.M3_ERR_INVALID_VALUE
    # partial overlap of h_in and h_out is rejected
    d = dims(b=2, n=16, p=16)
    assert call(d, h_in=ctypes.c_void_p(0x10000), h_out=ctypes.c_void_p(0x10010)) == \
        m3.M3_ERR_INVALID_VALUE


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not found"):
        _binding.load_library(str(tmp_path / "missing.so"))


def test_prefill_lds_limit(lib):
    """float32 with N=128, P=64 and chunk 128 needs more than 160 KB of LDS."""
    d = dims(t=256, p=64, n=128)
    fake = ctypes.c_void_p(0x10000)
    assert lib.m3_prefill(ctypes.byref(d), m3.M3_F32, 128, fake, fake, fake, fake, fake, fake,
                          fake, fake, None, fake, 1 << 40, None) == m3.M3_ERR_NOT_SUPPORTED
    assert ws(d, 128, m3.M3_F32) == 0
    assert ws(d, 64, m3.M3_F32) > 0


def test_block_pass_validation(lib):
    """Host-side checks of the block-side passes (nothing is launched)."""
    ok = ctypes.c_void_p(0x100000)
    mis16 = ctypes.c_void_p(0x100008)   # 8-byte aligned, not 16
    mis4 = ctypes.c_void_p(0x100002)

    def pre(d, ptrs=None, eps=1e-6, dtype=m3.M3_BF16):
        p = ptrs or [ok] * 11   # x B C nB nC bB bC up x_out B_out C_out
        return lib.m3_block_prepass(ctypes.byref(d), dtype, *p[:8], ctypes.c_float(eps), *p[8:],
                                    None)

    d = dims(b=2, t=8, h=2, p=64, n=64, r=2)
    assert pre(dims(n=48)) == m3.M3_ERR_NOT_SUPPORTED      # rows must be 2^k vectors
    assert pre(dims(n=512)) == m3.M3_ERR_NOT_SUPPORTED
    assert pre(dims(p=24)) == m3.M3_ERR_NOT_SUPPORTED
    assert pre(dims(r=3)) == m3.M3_ERR_NOT_SUPPORTED
    assert pre(d, dtype=9) == m3.M3_ERR_INVALID_VALUE
    assert pre(d, eps=-1.0) == m3.M3_ERR_INVALID_VALUE
    assert pre(d, eps=float("nan")) == m3.M3_ERR_INVALID_VALUE
    assert pre(dims(b=0)) == m3.M3_SUCCESS
    assert pre(dims(t=0)) == m3.M3_SUCCESS
    for i in range(11):
        p = [ok] * 11
        p[i] = None
        assert pre(d, p) == m3.M3_ERR_INVALID_VALUE
        p[i] = mis16 if i in (0, 1, 2, 8, 9, 10) else mis4
        assert pre(d, p) == m3.M3_ERR_INVALID_VALUE

    def post(d, y=ok, down=ok, out=ok):
        return lib.m3_block_postpass(ctypes.byref(d), m3.M3_F32, y, down, out, None)
    assert post(dims(b=0)) == m3.M3_SUCCESS
    assert post(d, y=None) == m3.M3_ERR_INVALID_VALUE
    assert post(d, y=mis16) == m3.M3_ERR_INVALID_VALUE
    assert post(d, down=mis4) == m3.M3_ERR_INVALID_VALUE
    assert post(d, out=None) == m3.M3_ERR_INVALID_VALUE
    assert post(dims(r=3)) == m3.M3_ERR_NOT_SUPPORTED


def test_backward_validation(lib):
    """Host-side checks of m3_backward (nothing is launched)."""
    ok = ctypes.c_void_p(0x100000)
    mis = ctypes.c_void_p(0x100001)

    def call(d, ptrs=None, dtype=m3.M3_F32, ws=ok, wsb=1 << 40):
        p = ptrs or [ok] * 16  # x dt A lam theta B C dy dh dx ddt dA dlam dtheta dB dC
        return lib.m3_backward(ctypes.byref(d), dtype, *p, ws, wsb, None)

    d = dims(b=2, t=16, h=2, p=64, n=64, r=2)
    assert call(dims(n=48)) == m3.M3_ERR_NOT_SUPPORTED     # power-of-two state size
    assert call(dims(n=256, p=64)) == m3.M3_ERR_NOT_SUPPORTED  # N * P > 8192
    assert call(dims(r=3)) == m3.M3_ERR_NOT_SUPPORTED
    assert call(d, dtype=7) == m3.M3_ERR_INVALID_VALUE
    for i in range(16):
        p = [ok] * 16
        if i != 8:  # dh_final is optional
            p[i] = None
            assert call(d, p) == m3.M3_ERR_INVALID_VALUE
        p[i] = mis
        assert call(d, p) == m3.M3_ERR_INVALID_VALUE
    assert call(d, ws=None) == m3.M3_ERR_WORKSPACE
    need = lib.m3_backward_workspace_size(ctypes.byref(d), m3.M3_F32)
    # N = P = 64: chunks of 64 / R = 32 tokens; per head the entry state of
    # every chunk and of the next (nC + 1 states), the exit adjoint of every
    # chunk (nC states), four partial scalars per token, 65 floats per chunk
    # (each area rounded up to 256 bytes)
    st = 64 * 64 * 4
    assert need == 4 * 2 * st + 4 * 1 * st + 4 * 4 * 16 * 4 + 1280
    d40 = dims(b=2, t=40, h=2, p=64, n=64, r=2)
    assert lib.m3_backward_workspace_size(ctypes.byref(d40), m3.M3_F32) == \
        4 * 3 * st + 4 * 2 * st + 4 * 4 * 40 * 4 + 2304
    # other N P <= 4096: segments (32 tokens here), one entry state and one
    # exit adjoint per segment and head; the dA terms; per segment a decay
    # and N / 2 angles
    d32 = dims(b=2, t=16, h=2, p=32, n=32, r=1)
    assert lib.m3_backward_workspace_size(ctypes.byref(d32), m3.M3_F32) == \
        2 * (2 * 2 * 1 * 32 * 32 * 4) + 256 + 256 + 256
    # N P = 8192: h_t and G_t of every token-head
    d8k = dims(b=2, t=16, h=2, p=64, n=128, r=1)
    assert lib.m3_backward_workspace_size(ctypes.byref(d8k), m3.M3_BF16) == \
        2 * (2 * 2 * 16 * 128 * 64 * 4) + 256
    assert call(d, wsb=need - 1) == m3.M3_ERR_WORKSPACE
    assert lib.m3_backward_workspace_size(ctypes.byref(dims(b=0)), m3.M3_F32) == 0
