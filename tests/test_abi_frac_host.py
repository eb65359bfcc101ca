"""Host-side checks of the learned-alpha (fractional entry) calls of libfsa: the
table against the oracle, argument validation and the workspace size, all
returning before any HIP call."""
import ctypes
import math

import numpy as np
import pytest

import oracle
from fibonacci_offset_transformer_amd import fsa

P = ctypes.c_void_p
FAKE = [P(0x10000 * (i + 1)) for i in range(14)]  # distinct, aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    return fsa.library()


def table(lib, base, alpha, w, R, capacity=fsa.MAX_OFFSETS):
    wh = (ctypes.c_int32 * max(capacity, 1))()
    fr = (ctypes.c_float * max(capacity, 1))()
    fb = (ctypes.c_int32 * max(capacity, 1))()
    cnt = ctypes.c_int32(-7)
    st = lib.fsa_frac_offsets(fsa.BASES[base], alpha, w, R, wh, fr, fb, capacity, ctypes.byref(cnt))
    n = min(cnt.value, capacity)
    return st, [(wh[i], fr[i], fb[i]) for i in range(n)] if st == 0 else None, cnt.value


@pytest.mark.parametrize("base", ["fib", "pow2"])
def test_frac_tables_match_oracle(lib, base):
    al = [0.5 + l / 15.0 for l in range(16)] + list(np.random.default_rng(7).uniform(0.5, 1.5, 300))
    al += [1.0, 0.5, 1.5, 2.0, 3.3]
    for a in al:
        for w in (1, 6, 8, 12, 64):
            for R in (1, 100, 1024, 4096):
                st, got, _ = table(lib, base, float(a), w, R)
                assert st == fsa.FSA_OK
                want = oracle.frac_offset_table(base, float(a), w, R)
                assert len(got) == len(want)
                for (wh, fr, fb), (d, f) in zip(got, want):
                    assert fb == f and wh == math.floor(d)
                    assert fr == float(np.float32(d - math.floor(d)))  # the float nearest phi


def test_frac_table_integer_alpha_is_the_static_table(lib):
    st, got, _ = table(lib, "fib", 1.0, 64, 1024)
    assert [(wh, fr) for wh, fr, _ in got] == [(o, 0.0) for o in fsa.build_offsets(1.0, 64, 1024)]


def test_frac_table_capacity_and_errors(lib):
    st, _, cnt = table(lib, "fib", 1.0, 1, 1024, capacity=3)
    assert st == fsa.FSA_E_CAPACITY and cnt == 15
    assert table(lib, "fib", 0.0, 8, 1024)[0] == fsa.FSA_E_ARG
    assert table(lib, "fib", 1.0, 0, 1024)[0] == fsa.FSA_E_ARG
    assert table(lib, "fib", 1.0, 8, 0)[0] == fsa.FSA_E_ARG
    assert table(lib, "fib", float("inf"), 8, 1024)[0] == fsa.FSA_E_ARG
    assert lib.fsa_frac_offsets(0, 1.0, 8, 1024, None, None, None, 0, None) == fsa.FSA_E_ARG
    cnt = ctypes.c_int32(0)
    assert lib.fsa_frac_offsets(0, 1.0, 8, 1024, None, None, None, 48, ctypes.byref(cnt)) == fsa.FSA_E_ARG


def ffwd(lib, dt=1, ptrs=None, B=1, H=1, N=64, d=64, scale=0.125, base=0, alpha=1.3, w=16, R=256, out_dt=1):
    p = ptrs or FAKE[:5]
    return lib.fsa_frac_forward(dt, out_dt, *p, B, H, N, d, scale, base, alpha, w, R, None)


def fbwd(lib, dt=1, ptrs=None, B=1, H=1, N=64, d=64, scale=0.125, base=0, alpha=1.3, w=16, R=256, out_dt=1,
         ws_bytes=1 << 40):
    p = ptrs or FAKE[:12]  # q k v o lse dout dq dk dv dalpha doffs ws
    return lib.fsa_frac_backward(dt, out_dt, *p, ws_bytes, B, H, N, d, scale, base, alpha, w, R, None)


@pytest.mark.parametrize("call", [ffwd, fbwd])
def test_frac_pair_words_need_32_bit_offsets(lib, call):
    # w = 1, R = 2^30: 35 entries below N = 2^24 (40 slots of four fp32 words below w = 64:
    # 10.7 GB per head)
    assert call(lib, N=1 << 24, w=1, R=1 << 30) == fsa.FSA_E_UNSUPPORTED
    assert b"32-bit pair offsets" in lib.fsa_last_error()
    # 12 entries (R = 300) take 16 slots: at N = 2^22 (1.07 GB per head) they are accepted,
    # at N = 2^23 (2.1 GB) not; at w = 64 (two words per slot) N = 2^23 fits
    ws = ctypes.c_uint64(0)
    assert lib.fsa_frac_backward_workspace_bytes(1, 1, 1, 1 << 22, 64, 0, 1.0, 1, 300, ctypes.byref(ws)) == 0
    assert ws.value > 16 * 16 << 22
    assert call(lib, N=1 << 23, w=1, R=300) == fsa.FSA_E_UNSUPPORTED
    assert lib.fsa_frac_backward_workspace_bytes(1, 1, 1, 1 << 23, 64, 0, 20.0, 64, 300, ctypes.byref(ws)) == 0


@pytest.mark.parametrize("call", [ffwd, fbwd])
def test_frac_shape_dtype_and_path_errors(lib, call):
    assert call(lib, d=32) == fsa.FSA_E_UNSUPPORTED
    assert call(lib, d=0) == fsa.FSA_E_ARG
    assert call(lib, dt=5) == fsa.FSA_E_UNSUPPORTED
    assert call(lib, B=-1) == fsa.FSA_E_ARG
    assert call(lib, scale=float("nan")) == fsa.FSA_E_ARG
    assert call(lib, alpha=0.0) == fsa.FSA_E_ARG
    assert call(lib, w=0) == fsa.FSA_E_ARG
    # valid but outside the implemented path
    assert call(lib, dt=0) == fsa.FSA_E_UNSUPPORTED and b"bf16" in lib.fsa_last_error()
    assert call(lib, w=65) == fsa.FSA_E_UNSUPPORTED and b"w <= 64" in lib.fsa_last_error()
    assert call(lib, scale=0.0) == fsa.FSA_E_UNSUPPORTED and b"positive" in lib.fsa_last_error()
    assert call(lib, scale=-0.1) == fsa.FSA_E_UNSUPPORTED
    assert call(lib, N=(1 << 24) + 1) == fsa.FSA_E_UNSUPPORTED


def test_frac_forward_pointer_checks(lib):
    for k in range(5):
        ptrs = list(FAKE[:5])
        ptrs[k] = P(0)
        assert ffwd(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"NULL" in lib.fsa_last_error()
        ptrs[k] = P(FAKE[k].value + 8)
        assert ffwd(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"aligned" in lib.fsa_last_error()
    ptrs = list(FAKE[:5])
    ptrs[3] = ptrs[1]
    assert ffwd(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"aliases" in lib.fsa_last_error()
    for B, H, N in ((0, 1, 64), (1, 0, 64), (1, 1, 0)):
        assert ffwd(lib, ptrs=[P(0)] * 5, B=B, H=H, N=N) == fsa.FSA_OK


def test_frac_backward_pointer_checks(lib):
    tensors = [0, 1, 2, 3, 4, 5, 6, 7, 8, 11]  # every argument but dalpha and doffs
    for k in tensors:
        ptrs = list(FAKE[:12])
        ptrs[k] = P(0)
        assert fbwd(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"NULL" in lib.fsa_last_error()
        ptrs[k] = P(FAKE[k].value + 8)
        assert fbwd(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"aligned" in lib.fsa_last_error()
    ptrs = list(FAKE[:12])
    ptrs[9] = P(0)
    assert fbwd(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"dalpha is NULL" in lib.fsa_last_error()
    ptrs[9] = P(FAKE[9].value + 2)
    assert fbwd(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"dalpha" in lib.fsa_last_error()
    ptrs = list(FAKE[:12])
    ptrs[10] = P(FAKE[10].value + 1)
    assert fbwd(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"doffs" in lib.fsa_last_error()
    for k, other in ((6, 0), (8, 5), (11, 3)):  # dq = q, dv = dout, ws = o
        ptrs = list(FAKE[:12])
        ptrs[k] = ptrs[other]
        assert fbwd(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"aliases" in lib.fsa_last_error()
    for k in (0, 6, 11):  # dalpha aliasing q, dq, ws
        ptrs = list(FAKE[:12])
        ptrs[9] = ptrs[k]
        assert fbwd(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"aliases" in lib.fsa_last_error()
    ptrs = list(FAKE[:12])
    ptrs[10] = ptrs[9]  # doffs aliasing dalpha
    assert fbwd(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"aliases" in lib.fsa_last_error()


def frac_ws(lib, dt=1, B=2, H=8, N=4096, d=64, base=0, alpha=1.0, w=64, R=1024):
    out = ctypes.c_uint64(123)
    st = lib.fsa_frac_backward_workspace_bytes(dt, B, H, N, d, base, alpha, w, R, ctypes.byref(out))
    return st, out.value


def a256(x):
    return (x + 255) // 256 * 256


def test_frac_workspace_size(lib):
    # D, the pair words (two per pair at w = 64, four below), the per-tile partials, then one 64-bit token per
    # tile (the one-launch backward) and the status word, each part rounded up to 256 bytes.
    # alpha = 1.3, w = 64, R = 1024: d = 1.3 F >= 64 for F = 55 .. 987 (7 entries) -> 8 slots
    bh, N = 16, 4096
    n_ent = len(oracle.frac_offset_table("fib", 1.3, 64, 1024))
    assert n_ent == 7
    want = a256(4 * bh * N) + a256(8 * 8 * bh * N) + a256(4 * bh * (N // 64) * n_ent) + a256(8 * bh * (N // 64)) + 256
    assert frac_ws(lib, alpha=1.3) == (fsa.FSA_OK, want)
    # entries whose first row (ceil d) is not below N are dropped: N = 200 keeps d = 71.5, 115.7, 187.2
    n = 200
    want = a256(4 * bh * n) + a256(8 * 8 * bh * n) + a256(4 * bh * 4 * 3) + a256(8 * bh * 4) + 256
    assert frac_ws(lib, alpha=1.3, N=n) == (fsa.FSA_OK, want)
    # 9 entries (w = 1, alpha = 1.1, R = 60) take 16 slots, of four fp32 words below w = 64
    assert len(oracle.frac_offset_table("fib", 1.1, 1, 60)) == 9
    want = a256(4 * bh * N) + a256(16 * 16 * bh * N) + a256(4 * bh * (N // 64) * 9) + a256(8 * bh * (N // 64)) + 256
    assert frac_ws(lib, alpha=1.1, w=1, R=60) == (fsa.FSA_OK, want)
    assert frac_ws(lib, B=0) == (fsa.FSA_OK, 0)
    assert frac_ws(lib, dt=0)[0] == fsa.FSA_E_UNSUPPORTED
    assert lib.fsa_frac_backward_workspace_bytes(1, 1, 1, 64, 64, 0, 1.0, 64, 1024, None) == fsa.FSA_E_ARG


def test_frac_backward_workspace_too_small(lib):
    st, need = frac_ws(lib, B=1, H=1, N=64, alpha=1.3, w=16, R=256)
    assert st == fsa.FSA_OK and need > 0
    assert fbwd(lib, ws_bytes=need - 1) == fsa.FSA_E_ARG and b"ws holds" in lib.fsa_last_error()


def fdec(lib, dt=1, ptrs=None, B=1, H=1, N=64, d=64, scale=0.125, base=0, alpha=1.3, w=16, R=256, out_dt=1):
    p = ptrs or FAKE[:6]  # q k_cache v_cache seq_lens o lse; N is Lmax
    return lib.fsa_frac_decode(dt, out_dt, *p, B, H, N, d, scale, base, alpha, w, R, None)


def test_frac_decode_checks(lib):
    assert fdec(lib, d=32) == fsa.FSA_E_UNSUPPORTED
    assert fdec(lib, alpha=0.0) == fsa.FSA_E_ARG
    assert fdec(lib, N=0) == fsa.FSA_E_ARG and b"Lmax" in lib.fsa_last_error()
    ptrs = list(FAKE[:6])
    ptrs[3] = P(0)
    assert fdec(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"seq_lens is NULL" in lib.fsa_last_error()
    ptrs[3] = P(FAKE[3].value + 2)
    assert fdec(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"4-byte" in lib.fsa_last_error()
    for k in (0, 1, 2, 4, 5):
        ptrs = list(FAKE[:6])
        ptrs[k] = P(0)
        assert fdec(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"NULL" in lib.fsa_last_error()
    ptrs = list(FAKE[:6])
    ptrs[5] = ptrs[2]
    assert fdec(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"aliases" in lib.fsa_last_error()
    assert fdec(lib, ptrs=[P(0)] * 6, B=0) == fsa.FSA_OK
