"""Host-side checks of libfsa that need no GPU: the library loads, exports every
symbol include/fsa.h declares, builds offset tables bit-exactly like the oracle,
and rejects every invalid argument before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from fibonacci_offset_transformer_amd import fsa, schedules

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return fsa.library()


def header_functions():
    text = open(os.path.join(ROOT, "include", "fsa.h")).read()
    return sorted(set(re.findall(r"\b(fsa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_bound_functions():
    assert header_functions() == sorted(fsa.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_exported_symbols_are_c_linkage():
    # nm -D lists the plain (unmangled) names
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", fsa._LIB_PATH], capture_output=True, text=True).stdout
    names = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in header_functions():
        assert name in names, name


def build(lib, base, alpha, w, R, capacity=fsa.MAX_OFFSETS):
    out = (ctypes.c_int32 * max(capacity, 1))()
    cnt = ctypes.c_int32(-7)
    st = lib.fsa_build_offsets(fsa.BASES[base], alpha, w, R, out, capacity, ctypes.byref(cnt))
    return st, [out[i] for i in range(min(cnt.value, capacity))] if st == 0 else None, cnt.value


def alphas():
    al = [0.5 + l / 15.0 for l in range(16)] + [0.5, 1.0, 1.5]
    al += list(np.random.default_rng(2024).uniform(0.5, 1.5, 1000))
    al += [0.25, 2.0, 3.7, 1e-3, 1e3]
    return [float(a) for a in al]


@pytest.mark.parametrize("base", ["fib", "pow2"])
def test_tables_bit_exact_against_oracle(lib, base):
    for a in alphas():
        for w in (1, 6, 8, 10, 12, 16, 64):
            for R in (1, 2, 256, 1024, 4096):
                st, got, _ = build(lib, base, a, w, R)
                assert st == fsa.FSA_OK
                assert got == oracle.offset_table(base, a, w, R), (base, a, w, R)


def test_golden_tables(lib):
    assert build(lib, "fib", 1.0, 16, 256)[1] == [21, 34, 55, 89, 144, 233]
    assert build(lib, "fib", 1.0, 64, 1024)[1] == [89, 144, 233, 377, 610, 987]
    assert build(lib, "pow2", 1.0, 64, 1024)[1] == [64, 128, 256, 512]
    assert build(lib, "fib", 1.0, 1, 1024)[1][:6] == [1, 2, 3, 5, 8, 13]


def test_stagger_alphas_match_oracle_schedule():
    ours = schedules.linear_stagger(16)
    assert ours == [oracle.stagger_alpha(l) for l in range(16)]  # bitwise-equal doubles
    assert schedules.coprime_stagger(16) == [ours[oracle.coprime_layer(l)] for l in range(16)]


def test_ties_round_half_even(lib):
    # alpha = 0.5: 0.5 * 233 = 116.5 -> 116 (even); 0.5 * 377 = 188.5 -> 188
    assert build(lib, "fib", 0.5, 64, 1024)[1] == [72, 116, 188, 305, 494]
    # alpha = 1.5: 1.5 * 987 = 1480.5 -> 1480
    assert build(lib, "fib", 1.5, 64, 1024)[1][-1] == 1480


def test_large_reach_and_max_table(lib):
    st, got, cnt = build(lib, "fib", 1.0, 1, 2**31 - 1)
    assert st == fsa.FSA_OK and got == oracle.offset_table("fib", 1.0, 1, 2**31 - 1)
    assert cnt <= fsa.MAX_OFFSETS


def test_capacity_error_reports_count(lib):
    st, _, cnt = build(lib, "fib", 1.0, 64, 1024, capacity=3)
    assert st == fsa.FSA_E_CAPACITY and cnt == 6
    assert b"capacity" in lib.fsa_last_error()
    st, _, cnt = build(lib, "fib", 1.0, 2000, 1024, capacity=0)  # empty table fits
    assert st == fsa.FSA_OK and cnt == 0


@pytest.mark.parametrize("base,alpha,w,R", [
    (0, 0.0, 64, 1024), (0, -1.0, 64, 1024), (0, float("nan"), 64, 1024), (0, float("inf"), 64, 1024),
    (0, 1.0, 0, 1024), (0, 1.0, -3, 1024), (0, 1.0, 64, 0), (0, 1.0, 64, -1), (7, 1.0, 64, 1024),
    (0, 3.0, 1, 2**31 - 1),      # alpha * F overflows int32
    (1, 1.0, 1, 2**31 - 1),      # fine: 2^30 * 1 fits ...
])
def test_build_offsets_argument_errors(lib, base, alpha, w, R):
    out = (ctypes.c_int32 * 48)()
    cnt = ctypes.c_int32(0)
    st = lib.fsa_build_offsets(base, alpha, w, R, out, 48, ctypes.byref(cnt))
    if (base, alpha, w, R) == (1, 1.0, 1, 2**31 - 1):
        assert st == fsa.FSA_OK
    else:
        assert st == fsa.FSA_E_ARG
        assert lib.fsa_last_error() != b""


def test_build_offsets_null_count(lib):
    out = (ctypes.c_int32 * 48)()
    assert lib.fsa_build_offsets(0, 1.0, 64, 1024, out, 48, None) == fsa.FSA_E_ARG


# ---- attention entry points: only paths that return before any HIP call ----

P = ctypes.c_void_p
FAKE = [P(0x10000 * (i + 1)) for i in range(12)]  # distinct, aligned, never dereferenced


def fwd(lib, dt=1, ptrs=None, B=1, H=1, N=64, d=64, scale=0.125, base=0, alpha=1.0, w=16, R=256, out_dt=1):
    p = ptrs or FAKE[:5]
    return lib.fsa_forward(dt, out_dt, *p, B, H, N, d, scale, base, alpha, w, R, None)


def bwd(lib, dt=1, ptrs=None, B=1, H=1, N=64, d=64, scale=0.125, base=0, alpha=1.0, w=16, R=256, out_dt=1,
        pair_bytes=1 << 40):
    p = ptrs or FAKE[:11]  # q k v o lse dout dq dk dv delta_ws pair_ws
    return lib.fsa_backward(dt, out_dt, *p, pair_bytes, B, H, N, d, scale, base, alpha, w, R, None)


def grads(lib, dt=1, ptrs=None, B=1, H=1, N=64, d=64, scale=0.125, base=0, alpha=1.0, w=16, R=256, out_dt=1,
          pair_bytes=1 << 40):
    p = ptrs or FAKE[:10]  # q k v lse dout delta dq dk dv pair_ws
    return lib.fsa_backward_grads(dt, out_dt, *p, pair_bytes, B, H, N, d, scale, base, alpha, w, R, None)


def decode(lib, dt=1, ptrs=None, B=1, H=1, N=64, d=64, scale=0.125, base=0, alpha=1.0, w=16, R=256, out_dt=1):
    p = ptrs or FAKE[:6]  # q k_cache v_cache seq_lens o lse; N is Lmax
    return lib.fsa_decode(dt, out_dt, *p, B, H, N, d, scale, base, alpha, w, R, None)


def dense(lib, dt=1, ptrs=None, B=1, H=1, N=64, d=64, scale=0.125, out_dt=1):
    p = ptrs or FAKE[:5]
    return lib.fsa_dense_forward(dt, out_dt, *p, B, H, N, d, scale, None)


@pytest.mark.parametrize("call", [fwd, bwd, grads, decode, dense])
def test_shape_and_dtype_errors(lib, call):
    assert call(lib, d=32) == fsa.FSA_E_UNSUPPORTED
    assert call(lib, d=0) == fsa.FSA_E_ARG
    assert call(lib, dt=5) == fsa.FSA_E_UNSUPPORTED
    assert call(lib, out_dt=3) == fsa.FSA_E_UNSUPPORTED
    assert call(lib, B=-1) == fsa.FSA_E_ARG
    assert call(lib, N=-5) == fsa.FSA_E_ARG
    assert call(lib, scale=float("nan")) == fsa.FSA_E_ARG
    assert call(lib, scale=float("inf")) == fsa.FSA_E_ARG
    assert call(lib, B=1 << 20, H=1 << 12, N=1 << 16) == fsa.FSA_E_ARG  # grid too large


@pytest.mark.parametrize("call", [fwd, bwd, grads, decode])
def test_table_errors_on_attention_calls(lib, call):
    assert call(lib, alpha=0.0) == fsa.FSA_E_ARG
    assert call(lib, alpha=float("nan")) == fsa.FSA_E_ARG
    assert call(lib, w=0) == fsa.FSA_E_ARG
    assert call(lib, R=0) == fsa.FSA_E_ARG
    assert call(lib, base=9) == fsa.FSA_E_ARG


@pytest.mark.parametrize("call,n", [(fwd, 5), (bwd, 11), (grads, 10), (dense, 5)])
def test_null_misaligned_and_aliased_pointers(lib, call, n):
    for k in range(n):
        ptrs = list(FAKE[:n])
        ptrs[k] = P(0)
        assert call(lib, ptrs=ptrs) == fsa.FSA_E_ARG
        assert b"NULL" in lib.fsa_last_error()
        ptrs[k] = P(FAKE[k].value + 8)
        assert call(lib, ptrs=ptrs) == fsa.FSA_E_ARG
        assert b"aligned" in lib.fsa_last_error()
    ptrs = list(FAKE[:n])
    ptrs[n - 1] = ptrs[0]  # an output aliasing q
    assert call(lib, ptrs=ptrs) == fsa.FSA_E_ARG
    assert b"aliases" in lib.fsa_last_error()


@pytest.mark.parametrize("call,n", [(fwd, 5), (bwd, 11), (grads, 10), (dense, 5)])
def test_empty_problems_launch_nothing(lib, call, n):
    nulls = [P(0)] * n
    for B, H, N in ((0, 1, 64), (1, 0, 64), (1, 1, 0)):
        assert call(lib, ptrs=nulls, B=B, H=H, N=N) == fsa.FSA_OK
        assert lib.fsa_last_error() == b""


def ws_bytes(lib, dt=1, B=2, H=8, N=4096, d=64, base=0, alpha=1.0, w=64, R=1024):
    out = ctypes.c_uint64(123)
    st = lib.fsa_backward_workspace_bytes(dt, B, H, N, d, base, alpha, w, R, ctypes.byref(out))
    return st, out.value


def a256(x):
    return (x + 255) // 256 * 256


def pair_ws(words, bh, n):
    # the pair words, then (256-byte aligned) one 64-bit completion token per 64-row tile,
    # then the 8-byte status word
    return a256(4 * words) + 8 * bh * ((n + 63) // 64) + 8


def test_backward_workspace_size(lib):
    # bf16, window 64: one 32-bit word per (head, row, offset slot), slots rounded up to
    # a multiple of 8; alpha = 1, R = 1024 gives the offsets 89, 144, 233, 377, 610, 987
    assert ws_bytes(lib) == (fsa.FSA_OK, pair_ws(8 * 16 * 4096, 16, 4096))
    assert pair_ws(8 * 16 * 4096, 16, 4096) == 4 * 8 * 16 * 4096 + 8 * 16 * 64 + 8
    # offsets >= N are dropped: at N = 600 only 89, 144, 233, 377 remain (still 8 slots)
    assert ws_bytes(lib, N=600) == (fsa.FSA_OK, pair_ws(8 * 16 * 600, 16, 600))
    # narrower windows carry each pair as two fp32 words: a table of 9 offsets takes 16
    # slots (w = 1, alpha = 1, R = 60 gives 1, 2, 3, 5, 8, 13, 21, 34, 55)
    assert ws_bytes(lib, w=1, R=60) == (fsa.FSA_OK, pair_ws(2 * 16 * 16 * 4096, 16, 4096))
    assert ws_bytes(lib, w=63) == (fsa.FSA_OK, pair_ws(2 * 8 * 16 * 4096, 16, 4096))
    # an odd row count (offset 89 only): the token area starts 256-byte aligned
    assert ws_bytes(lib, B=1, H=3, N=101) == (fsa.FSA_OK, pair_ws(8 * 3 * 101, 3, 101))
    # no offset below N: no slots
    assert ws_bytes(lib, N=50, alpha=1.0, w=64) == (fsa.FSA_OK, 0)
    # paths without the pair workspace: fp32 inputs, wide windows
    assert ws_bytes(lib, dt=0) == (fsa.FSA_OK, 0)
    assert ws_bytes(lib, w=65) == (fsa.FSA_OK, 0)
    assert ws_bytes(lib, B=0) == (fsa.FSA_OK, 0)
    assert ws_bytes(lib, alpha=0.0)[0] == fsa.FSA_E_ARG
    assert ws_bytes(lib, d=32)[0] == fsa.FSA_E_UNSUPPORTED
    assert lib.fsa_backward_workspace_bytes(1, 1, 1, 64, 64, 0, 1.0, 64, 1024, None) == fsa.FSA_E_ARG


def test_backward_pair_words_need_32_bit_offsets(lib):
    # w = 1, R = 2^30: the Fibonacci numbers below N are all offsets, each pair two words.
    # At N = 2^22 there are 31 (32 slots, 256 bytes per row: 1 GiB per head, within
    # 32-bit offsets); at N = 2^23, 33 (40 slots: 2.7 GB per head), so the backward takes
    # the general kernels, which need no pair words
    n22 = 1 << 22
    assert ws_bytes(lib, B=1, H=1, N=n22, w=1, R=1 << 30) == (fsa.FSA_OK, pair_ws(2 * 32 * n22, 1, n22))
    assert ws_bytes(lib, B=1, H=1, N=1 << 23, w=1, R=1 << 30) == (fsa.FSA_OK, 0)
    # with w = 64 (one word per pair) 2^24 rows of 8 slots still fit
    n24 = 1 << 24
    assert ws_bytes(lib, B=1, H=1, N=n24, w=64, R=1 << 16) == (fsa.FSA_OK, pair_ws(16 * n24, 1, n24))


@pytest.mark.parametrize("call", [bwd, grads])
def test_backward_pair_workspace_checks(lib, call):
    # bf16, w = 16, N = 64, alpha = 1, R = 256: offsets 21, 34, 55 -> 8 slots of two words
    # * 64 rows, then one token for the single tile and the status word. Only failing
    # validations are exercised here (the pointers are fake); the calls that pass NULL for
    # an unneeded workspace run in the GPU tests (fp32 inputs).
    need = pair_ws(2 * 8 * 64, 1, 64)
    assert call(lib, pair_bytes=need - 1) == fsa.FSA_E_ARG
    assert b"pair_ws holds" in lib.fsa_last_error()
    assert call(lib, pair_bytes=0) == fsa.FSA_E_ARG
    n = 11 if call is bwd else 10
    ptrs = list(FAKE[:n])
    ptrs[n - 1] = P(0)
    assert call(lib, ptrs=ptrs) == fsa.FSA_E_ARG
    assert b"pair_ws is NULL" in lib.fsa_last_error()


def test_decode_specific_checks(lib):
    assert decode(lib, N=0) == fsa.FSA_E_ARG  # the cache holds at least the newest token
    assert b"Lmax" in lib.fsa_last_error()
    ptrs = list(FAKE[:6])
    ptrs[3] = P(0)
    assert decode(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"seq_lens is NULL" in lib.fsa_last_error()
    ptrs[3] = P(FAKE[3].value + 2)
    assert decode(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"4-byte" in lib.fsa_last_error()
    for k in (0, 1, 2, 4, 5):
        ptrs = list(FAKE[:6])
        ptrs[k] = P(0)
        assert decode(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"NULL" in lib.fsa_last_error()
        ptrs[k] = P(FAKE[k].value + 8)
        assert decode(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"aligned" in lib.fsa_last_error()
    ptrs = list(FAKE[:6])
    ptrs[4] = ptrs[1]  # o aliases the key cache
    assert decode(lib, ptrs=ptrs) == fsa.FSA_E_ARG and b"aliases" in lib.fsa_last_error()
    # empty batches launch nothing, whatever the pointers
    assert decode(lib, ptrs=[P(0)] * 6, B=0) == fsa.FSA_OK
    assert decode(lib, ptrs=[P(0)] * 6, H=0) == fsa.FSA_OK


def test_literal_stagger_tables(lib):
    # the literal formula reaches alpha = 2.0: eight offsets at the last two layers, the largest 1974
    al = schedules.literal_stagger(16)
    assert al[0] == 0.5 and al[15] == 2.0
    tabs = [build(lib, "fib", a, 64, 1024)[1] for a in al]
    assert tabs == [oracle.offset_table("fib", a, 64, 1024) for a in al]
    assert [len(t) for t in tabs][-2:] == [8, 8] and max(max(t) for t in tabs) == 1974


# ---- the wait-status call: argument checks and the paths without waits (no HIP call) ----

def wait_status(lib, kind=0, dt=1, B=2, H=4, N=300, d=64, base=0, alpha=1.0, w=64, R=1024, ws=None,
                ws_bytes=1 << 40, flag=True):
    out = ctypes.c_int32(7)
    st = lib.fsa_wait_status(kind, dt, B, H, N, d, base, alpha, w, R, ws if ws is not None else FAKE[0], ws_bytes,
                             ctypes.byref(out) if flag else None, None)
    return st, out.value


def test_wait_status_checks(lib):
    assert wait_status(lib, flag=False)[0] == fsa.FSA_E_ARG
    assert wait_status(lib, kind=9)[0] == fsa.FSA_E_ARG
    assert wait_status(lib, d=32)[0] == fsa.FSA_E_UNSUPPORTED
    assert wait_status(lib, alpha=0.0)[0] == fsa.FSA_E_ARG
    # one-launch shapes (B * H a multiple of 8) check the workspace before reading it
    assert wait_status(lib, ws=P(0))[0] == fsa.FSA_E_ARG
    assert wait_status(lib, ws_bytes=16)[0] == fsa.FSA_E_ARG and b"ws holds" in lib.fsa_last_error()
    # shapes that run without waits report 0 and read nothing
    assert wait_status(lib, B=1, H=3, ws=P(0)) == (fsa.FSA_OK, 0)        # two kernels
    assert wait_status(lib, N=50, ws=P(0)) == (fsa.FSA_OK, 0)            # no offset below N
    assert wait_status(lib, dt=0, ws=P(0)) == (fsa.FSA_OK, 0)            # fp32: general kernel
    assert wait_status(lib, kind=1, B=1, H=3, alpha=1.3, ws=P(0)) == (fsa.FSA_OK, 0)
    assert wait_status(lib, kind=2, B=1, H=3, ws=P(0)) == (fsa.FSA_OK, 0)
    assert wait_status(lib, kind=3, B=1, H=3, alpha=1.3, ws=P(0)) == (fsa.FSA_OK, 0)
    # the rotary forward waits (it rotates K in the kernel) only with B * H a multiple of 8
    assert wait_status(lib, kind=5, B=1, H=3, ws=P(0)) == (fsa.FSA_OK, 0)
    assert wait_status(lib, kind=5, ws=P(0))[0] == fsa.FSA_E_ARG
    assert wait_status(lib, kind=5, ws_bytes=16)[0] == fsa.FSA_E_ARG and b"ws holds" in lib.fsa_last_error()
    assert wait_status(lib, kind=5, d=32)[0] == fsa.FSA_E_UNSUPPORTED


def test_debug_force_wait_timeout_toggles(lib):
    assert lib.fsa_debug_force_wait_timeout(1) == fsa.FSA_OK
    assert lib.fsa_debug_force_wait_timeout(0) == fsa.FSA_OK


# ------------------------------------------------------------- workgroup order of the window kernels

def test_tile_order_rejects_bad_arguments(lib):
    assert lib.fsa_debug_tile_order(-1, None) == 1
    assert lib.fsa_debug_tile_order(5, None) == 1
    assert lib.fsa_debug_tile_order(0, None) == 0


@pytest.mark.parametrize("bh,N", [(16, 4096), (8, 4096), (64, 1024), (8, 32768), (8, 65), (24, 300),
                                  (3, 4096), (1, 100), (5, 257), (12, 1000)])
def test_tile_order_properties(bh, N):
    """The dispatch assumptions the one-launch waits rest on, checked on the order the
    kernels use: workgroup b (on XCD b mod 8, dispatched in increasing b) takes the
    logical tile order[b]. Every XCD gets one contiguous range of tiles in increasing
    order; with B * H a multiple of 8 that range is whole heads, so every tile a
    workgroup waits for (its own head's earlier tiles in the rotary forward; its head's
    dQ tiles in the one-launch backward, whose dK/dV grid follows the dQ grid) was
    dispatched earlier on the same XCD."""
    nt = (N + 63) // 64
    tiles = bh * nt
    order = fsa.debug_tile_order(tiles)
    assert sorted(order) == list(range(tiles))  # a permutation
    block_of = {t: b for b, t in enumerate(order)}
    for x in range(8):
        mine = [order[b] for b in range(x, tiles, 8)]
        if mine:
            assert mine == list(range(mine[0], mine[0] + len(mine)))  # contiguous, increasing
    if bh % 8:
        return
    for h in range(bh):
        xcds = {block_of[h * nt + t] % 8 for t in range(nt)}
        assert len(xcds) == 1  # whole heads per XCD
        blocks = [block_of[h * nt + t] for t in range(nt)]
        assert blocks == sorted(blocks)  # earlier tiles dispatched earlier
    # one-launch backward: dK/dV block tiles + b' takes tile order[b'] and waits for dQ
    # tiles of the same head; those sit on the same XCD and come earlier in the grid
    assert tiles % 8 == 0
    for b2 in range(tiles):
        t = order[b2]
        h = t // nt
        for t2 in range(t - t % nt, (h + 1) * nt):
            assert block_of[t2] % 8 == (tiles + b2) % 8 and block_of[t2] < tiles + b2
