"""Host-side checks of the rotary calls of libfsa: the table against the oracle's
(bit for bit), argument validation and workspace sizes, all returning before any
HIP call."""
import ctypes

import numpy as np
import pytest

import oracle
from fibonacci_offset_transformer_amd import fsa

P = ctypes.c_void_p
FAKE = [P(0x10000 * (i + 1)) for i in range(14)]  # distinct, aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    return fsa.library()


@pytest.mark.parametrize("n_pos,d,base", [(1, 64, 10000.0), (4096, 64, 10000.0), (300, 8, 10000.0),
                                          (100, 64, 500000.0), (33, 2, 10.0)])
def test_table_bit_exact_against_oracle(n_pos, d, base):
    t = fsa.rope_table(n_pos, d, base).numpy()
    assert np.array_equal(t, oracle.rope_table_f32(n_pos, d, base))


def test_table_errors(lib):
    buf = (ctypes.c_float * 64)()
    assert lib.fsa_rope_table(-1, 64, 10000.0, buf) == fsa.FSA_E_ARG
    assert lib.fsa_rope_table(1, 63, 10000.0, buf) == fsa.FSA_E_ARG
    assert lib.fsa_rope_table(1, 0, 10000.0, buf) == fsa.FSA_E_ARG
    assert lib.fsa_rope_table(1, 64, 0.0, buf) == fsa.FSA_E_ARG
    assert lib.fsa_rope_table(1, 64, float("nan"), buf) == fsa.FSA_E_ARG
    assert lib.fsa_rope_table(1, 64, 10000.0, None) == fsa.FSA_E_ARG
    assert lib.fsa_rope_table(0, 64, 10000.0, None) == fsa.FSA_OK


def rot(lib, dt=1, ptrs=None, n_pos=64, B=1, H=1, N=64, d=64):
    p = ptrs or FAKE[:3]  # x rope out
    return lib.fsa_rope_rotate(dt, p[0], p[1], n_pos, p[2], B, H, N, d, None)


def rfwd(lib, dt=1, ptrs=None, n_pos=64, B=1, H=1, N=64, d=64, scale=0.125, base=0, alpha=1.0, w=16, R=256,
         out_dt=1, ws_bytes=1 << 40):
    p = ptrs or FAKE[:7]  # q k v rope o lse ws
    return lib.fsa_rope_forward(dt, out_dt, p[0], p[1], p[2], p[3], n_pos, p[4], p[5], p[6], ws_bytes, 1,
                                B, H, N, d, scale, base, alpha, w, R, None)


def rbwd(lib, dt=1, ptrs=None, n_pos=64, B=1, H=1, N=64, d=64, scale=0.125, base=0, alpha=1.0, w=16, R=256,
         out_dt=1, ws_bytes=1 << 40):
    p = ptrs or FAKE[:11]  # q k v rope o lse dout dq dk dv ws
    return lib.fsa_rope_backward(dt, out_dt, p[0], p[1], p[2], p[3], n_pos, *p[4:10], p[10], ws_bytes, 0,
                                 B, H, N, d, scale, base, alpha, w, R, None)


def test_rotate_checks(lib):
    assert rot(lib, dt=0) == fsa.FSA_E_UNSUPPORTED
    assert rot(lib, N=(1 << 24) + 1, n_pos=(1 << 24) + 1) == fsa.FSA_E_UNSUPPORTED
    assert rot(lib, d=32) == fsa.FSA_E_UNSUPPORTED
    assert rot(lib, n_pos=63) == fsa.FSA_E_ARG and b"positions" in lib.fsa_last_error()
    for k in range(3):
        ptrs = list(FAKE[:3])
        ptrs[k] = P(0)
        assert rot(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"NULL" in lib.fsa_last_error()
        ptrs[k] = P(FAKE[k].value + 4)
        assert rot(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"aligned" in lib.fsa_last_error()
    assert rot(lib, ptrs=[FAKE[0], FAKE[1], FAKE[0]]) == fsa.FSA_E_ARG and b"aliases" in lib.fsa_last_error()
    assert rot(lib, ptrs=[P(0)] * 3, B=0) == fsa.FSA_OK


@pytest.mark.parametrize("call,n", [(rfwd, 7), (rbwd, 11)])
def test_rope_attention_checks(lib, call, n):
    assert call(lib, d=32) == fsa.FSA_E_UNSUPPORTED
    assert call(lib, dt=0) == fsa.FSA_E_UNSUPPORTED and b"bf16" in lib.fsa_last_error()
    assert call(lib, w=65) == fsa.FSA_E_UNSUPPORTED
    assert call(lib, scale=0.0) == fsa.FSA_E_UNSUPPORTED
    assert call(lib, N=(1 << 24) + 1, n_pos=(1 << 24) + 1) == fsa.FSA_E_UNSUPPORTED
    assert call(lib, n_pos=63) == fsa.FSA_E_ARG and b"positions" in lib.fsa_last_error()
    assert call(lib, alpha=0.0) == fsa.FSA_E_ARG
    assert call(lib, scale=float("nan")) == fsa.FSA_E_ARG
    for k in range(n):
        ptrs = list(FAKE[:n])
        ptrs[k] = P(0)
        assert call(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"NULL" in lib.fsa_last_error()
        ptrs[k] = P(FAKE[k].value + 8)
        assert call(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"aligned" in lib.fsa_last_error()
    ptrs = list(FAKE[:n])
    ptrs[n - 1] = ptrs[0]  # ws aliasing q
    assert call(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"aliases" in lib.fsa_last_error()
    assert call(lib, ptrs=[P(0)] * n, B=0) == fsa.FSA_OK
    assert call(lib, ws_bytes=0) == fsa.FSA_E_ARG and b"ws holds" in lib.fsa_last_error()


@pytest.mark.parametrize("call,n", [(rfwd, 7), (rbwd, 11)])
def test_rope_pair_words_need_32_bit_offsets(lib, call, n):
    # w = 1, R = 2^30: 43 offsets (48 slots: 3.2 GB of pair words per head at N = 2^24)
    assert call(lib, N=1 << 24, n_pos=1 << 24, w=1, R=1 << 30) == fsa.FSA_E_UNSUPPORTED
    assert b"32-bit pair offsets" in lib.fsa_last_error()


def a256(x):
    return (x + 255) // 256 * 256


def test_rope_workspace_sizes(lib):
    f, b = ctypes.c_uint64(1), ctypes.c_uint64(1)
    assert lib.fsa_rope_workspace_bytes(1, 2, 8, 4096, 64, 0, 1.0, 64, 1024, ctypes.byref(f), ctypes.byref(b)) == 0
    rows = 2 * 8 * 4096
    # rotated Q and K, then one 64-bit token per 64-row tile and the status word (the
    # forward that rotates K itself)
    fwd = 2 * a256(rows * 128) + a256(8 * 16 * 64 + 8)
    assert f.value == fwd
    # six offsets at alpha = 1, w = 64, R = 1024 -> 8 slots, then one 64-bit token per tile
    # and the status word
    pair = a256(4 * 8 * rows) + 8 * 16 * 64 + 8
    assert b.value == fwd + a256(4 * rows) + a256(pair)
    # a narrower window carries each pair as two words: w = 16 at N = 64 (offsets 21, 34, 55)
    assert lib.fsa_rope_workspace_bytes(1, 1, 2, 64, 64, 0, 1.0, 16, 256, ctypes.byref(f), ctypes.byref(b)) == 0
    rows = 2 * 64
    assert b.value == 2 * a256(rows * 128) + a256(8 * 2 + 8) + a256(4 * rows) + a256(a256(8 * 8 * rows) + 8 * 2 + 8)
    assert lib.fsa_rope_workspace_bytes(1, 0, 8, 4096, 64, 0, 1.0, 64, 1024, ctypes.byref(f), ctypes.byref(b)) == 0
    assert f.value == 0 and b.value == 0
    assert lib.fsa_rope_workspace_bytes(0, 1, 1, 64, 64, 0, 1.0, 64, 1024, ctypes.byref(f), ctypes.byref(b)) \
        == fsa.FSA_E_UNSUPPORTED
    assert lib.fsa_rope_workspace_bytes(1, 1, 1, 64, 64, 0, 1.0, 64, 1024, None, ctypes.byref(b)) == fsa.FSA_E_ARG


def rfrac_fwd(lib, ptrs=None, n_pos=64, N=64, dt=1, w=16, scale=0.125, ws_bytes=1 << 40):
    p = ptrs or FAKE[:7]  # q k v rope o lse ws
    return lib.fsa_rope_frac_forward(dt, 1, p[0], p[1], p[2], p[3], n_pos, p[4], p[5], p[6], ws_bytes,
                                     1, 1, N, 64, scale, 0, 1.3, w, 256, None)


def rfrac_bwd(lib, ptrs=None, n_pos=64, N=64, dt=1, w=16, scale=0.125, ws_bytes=1 << 40, B=1):
    p = ptrs or FAKE[:13]  # q k v rope o lse dout dq dk dv dalpha doffs ws
    return lib.fsa_rope_frac_backward(dt, 1, p[0], p[1], p[2], p[3], n_pos, *p[4:12], p[12], ws_bytes, 0,
                                      B, 1, N, 64, scale, 0, 1.3, w, 256, None)


@pytest.mark.parametrize("call,n", [(rfrac_fwd, 7), (rfrac_bwd, 13)])
def test_rope_frac_checks(lib, call, n):
    assert call(lib, dt=0) == fsa.FSA_E_UNSUPPORTED
    assert call(lib, w=65) == fsa.FSA_E_UNSUPPORTED
    assert call(lib, scale=0.0) == fsa.FSA_E_UNSUPPORTED
    assert call(lib, n_pos=63) == fsa.FSA_E_ARG and b"positions" in lib.fsa_last_error()
    assert call(lib, ws_bytes=0) == fsa.FSA_E_ARG and b"ws holds" in lib.fsa_last_error()
    skip = {10, 11} if n == 13 else set()  # dalpha and doffs have their own checks
    for k in range(n):
        if k in skip:
            continue
        ptrs = list(FAKE[:n])
        ptrs[k] = P(0)
        assert call(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"NULL" in lib.fsa_last_error()
        ptrs[k] = P(FAKE[k].value + 8)
        assert call(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"aligned" in lib.fsa_last_error()
    if n == 13:
        ptrs = list(FAKE[:13])
        ptrs[10] = P(0)
        assert call(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"dalpha is NULL" in lib.fsa_last_error()
        ptrs[10] = ptrs[0]
        assert call(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"aliases" in lib.fsa_last_error()


def test_rope_frac_workspace_sizes(lib):
    f, b = ctypes.c_uint64(1), ctypes.c_uint64(1)
    assert lib.fsa_rope_frac_workspace_bytes(1, 2, 8, 4096, 64, 0, 1.3, 64, 1024, ctypes.byref(f),
                                             ctypes.byref(b)) == 0
    rows = 2 * 8 * 4096
    fr = ctypes.c_uint64(0)
    assert lib.fsa_frac_backward_workspace_bytes(1, 2, 8, 4096, 64, 0, 1.3, 64, 1024, ctypes.byref(fr)) == 0
    assert f.value == 2 * a256(rows * 128) and b.value == f.value + fr.value
