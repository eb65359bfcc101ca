"""Pins of the oracle's rotary position embedding (the fused prologue).

The pages fix only that queries and keys are rotated before the rows are gathered
and that the rotation is vanilla RoPE without scaling (explainer page "Depth-
Staggered Fibonacci Spacing for Sparse Attention: Static Schedules Beat Learned
Dilation and Extrapolate Where Dense Attention Fails", Portuguese edition,
sections "Metodologia / Arquitetura", item "Implementação", and the limitations).
Each pin compares the oracle with something independent of its code:
  * complex multiplication (numpy): pair m as x_2m + i x_2m+1 times e^{i p theta_m};
  * the defining property of rotary embeddings: a query-key score depends on the
    two positions only through their difference;
  * closed forms for the frequencies; exact inverses and norm preservation;
  * central differences and torch autograd for the gradients through the rotation.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fsa_ref


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_frequencies_closed_form():
    ang = oracle.rope_angles(5, 64)
    assert ang.shape == (5, 32)
    assert np.all(ang[0] == 0.0)
    assert ang[1, 0] == 1.0                       # theta_0 = 1
    assert math.isclose(ang[1, 31], 10000.0 ** (-62 / 64), rel_tol=1e-15)
    assert math.isclose(ang[1, 16], 0.01, rel_tol=1e-14)   # 10000^(-1/2)
    assert np.allclose(ang[4], 4 * ang[1], rtol=1e-15)


def test_rotation_is_complex_multiplication():
    x = rand((3, 40, 64), 1)
    r = oracle.rope_rotate(x)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    pos = np.arange(40)[:, None]
    theta = 10000.0 ** (-np.arange(32) * 2.0 / 64)
    zr = z * np.exp(1j * pos * theta[None, :])
    assert np.max(np.abs(r[..., 0::2] - zr.real)) <= 1e-12
    assert np.max(np.abs(r[..., 1::2] - zr.imag)) <= 1e-12


def test_inverse_norms_and_position_zero():
    x = rand((2, 33, 64), 2)
    r = oracle.rope_rotate(x)
    assert np.max(np.abs(oracle.rope_rotate(r, inverse=True) - x)) <= 1e-12
    assert np.allclose(r[..., 0::2] ** 2 + r[..., 1::2] ** 2, x[..., 0::2] ** 2 + x[..., 1::2] ** 2, atol=1e-12)
    assert np.array_equal(r[:, 0], x[:, 0])


def test_scores_depend_on_relative_position_only():
    # the same query vector at every position and the same key vector at every position:
    # the rotated score of (i, j) equals that of (i + s, j + s)
    a, b = rand((64,), 3), rand((64,), 4)
    N = 50
    qr = oracle.rope_rotate(np.tile(a, (N, 1)))
    kr = oracle.rope_rotate(np.tile(b, (N, 1)))
    S = qr @ kr.T
    for i, j, s in ((10, 3, 7), (20, 20, 29), (5, 0, 44), (30, 12, 1)):
        assert abs(S[i, j] - S[i + s, j + s]) <= 1e-10
    assert abs(S[10, 3] - S[10, 4]) > 1e-3  # and it does depend on the difference


def test_forward_is_sparse_forward_on_rotated_rows():
    N, T, w = 120, [8, 13, 21, 34, 55, 89], 6
    q, k, v = (rand((2, N, 64), s) for s in (5, 6, 7))
    o, l = oracle.rope_sparse_forward(q, k, v, T, w, 0.125)
    z = lambda x: oracle.rope_rotate(x)
    o2, l2 = oracle.sparse_forward(z(q), z(k), v, T, w, 0.125)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)
    rows = np.array([0, 1, 7, 8, 60, 119])
    orow, lrow = oracle.rope_sparse_forward_rows(q, k, v, T, w, 0.125, rows)
    assert np.max(np.abs(orow - o[:, rows])) <= 1e-13 and np.max(np.abs(lrow - l[:, rows])) <= 1e-13


def _loss(q, k, v, do, T, w, scale):
    o, _ = oracle.rope_sparse_forward(q, k, v, T, w, scale)
    return float(np.sum(o * do))


def test_backward_matches_central_differences():
    N, d, T, w, scale = 14, 8, [3, 5, 8], 2, 0.6
    q, k, v, do = (rand((N, d), s) for s in (8, 9, 10, 11))
    dq, dk, dv = oracle.rope_sparse_backward(q, k, v, do, T, w, scale)
    h = 1e-6
    for X, G in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            old = X[idx]
            X[idx] = old + h
            lp = _loss(q, k, v, do, T, w, scale)
            X[idx] = old - h
            lm = _loss(q, k, v, do, T, w, scale)
            X[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        assert np.max(np.abs(num - G)) / max(1.0, np.max(np.abs(G))) <= 1e-6


def test_backward_matches_torch_autograd():
    # rotation written with torch complex numbers, attention as a masked dense softmax
    B, H, N, d, T, w, scale = 1, 2, 60, 16, [5, 8, 13, 21], 4, 0.25
    q, k, v, do = (rand((B, H, N, d), s) for s in (12, 13, 14, 15))
    dq, dk, dv = oracle.rope_sparse_backward(q, k, v, do, T, w, scale)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    pos = torch.arange(N, dtype=torch.float64)[:, None]
    theta = 10000.0 ** (-torch.arange(d // 2, dtype=torch.float64) * 2 / d)
    rot = torch.polar(torch.ones(N, d // 2, dtype=torch.float64), pos * theta)

    def rotate(x):
        z = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous())
        return torch.view_as_real(z * rot).reshape(x.shape)

    offs = set(range(w)) | set(T)
    M = torch.tensor([[(j <= i) and (i - j) in offs for j in range(N)] for i in range(N)])
    S = scale * (rotate(qt) @ rotate(kt).transpose(-1, -2))
    o = torch.softmax(S.masked_fill(~M, float("-inf")), dim=-1) @ vt
    o.backward(torch.from_numpy(do))
    for g, gt in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        assert np.max(np.abs(g - gt.numpy())) <= 1e-11


def test_backward_rows_match_full():
    N, T, w = 130, [8, 13, 21, 34, 55, 89], 6
    q, k, v, do = (rand((2, N, 64), s) for s in (16, 17, 18, 19))
    dq, dk, dv = oracle.rope_sparse_backward(q, k, v, do, T, w, 0.125)
    rows = np.array([0, 1, 5, 40, 100, 129])
    rq, rk, rv = oracle.rope_sparse_backward_rows(q, k, v, do, T, w, 0.125, rows)
    for a, b in ((rq, dq), (rk, dk), (rv, dv)):
        assert np.max(np.abs(a - b[:, rows])) <= 1e-12


# ---- planted mistakes ----

def _rotate_half_pairs(x, base=10000.0, inverse=False):
    # pairs (m, m + d/2) instead of (2m, 2m + 1)
    x = np.asarray(x, dtype=np.float64)
    N, d = x.shape[-2], x.shape[-1]
    ang = fsa_ref.rope_angles(N, d, base)
    c, s = np.cos(ang), np.sin(ang) * (-1 if inverse else 1)
    a, b = x[..., : d // 2], x[..., d // 2 :]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def _negative_angle(x, base=10000.0, inverse=False):
    return fsa_ref.__dict__["_orig_rotate"](x, base, inverse=not inverse)


@pytest.mark.parametrize("bad", [_rotate_half_pairs, _negative_angle])
def test_planted_rotation_mistakes_are_caught(monkeypatch, bad):
    monkeypatch.setitem(fsa_ref.__dict__, "_orig_rotate", fsa_ref.rope_rotate)
    monkeypatch.setattr(fsa_ref, "rope_rotate", bad)
    x = rand((3, 40, 64), 1)
    r = fsa_ref.rope_rotate(x)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    theta = 10000.0 ** (-np.arange(32) * 2.0 / 64)
    zr = z * np.exp(1j * np.arange(40)[:, None] * theta[None, :])
    assert np.max(np.abs(r[..., 0::2] - zr.real)) > 1e-3


# ---- the stored (bf16) rotation the fused path hands to the attention ----

def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_table_matches_numpy_cos_sin_to_a_float_ulp():
    tab = oracle.rope_table_f32(300, 64)
    ang = oracle.rope_angles(300, 64)
    for k, f in ((0, np.cos), (1, np.sin)):
        ref = f(ang).astype(np.float32)
        ulp = np.spacing(np.abs(ref)).astype(np.float64)
        assert np.all(np.abs(tab[..., k].astype(np.float64) - ref) <= ulp)


def test_stored_rotation_within_bf16_rounding_of_the_exact_one():
    x = _bf16(rand((2, 200, 64), 20))
    st = oracle.rope_store_bf16(x)
    ex = oracle.rope_rotate(x)
    assert np.array_equal(st, _bf16(st))  # bf16 values
    assert np.all(np.abs(st - ex) <= 2.0 ** -8 * np.abs(ex))  # half a bf16 step
    assert np.array_equal(st[:, 0], x[:, 0])  # position 0: cos 1, sin 0, nothing moves


def test_bf16_round_matches_torch_on_float32_values_and_ties():
    # for values that float32 holds exactly, torch's float32 -> bfloat16 conversion
    # (nearest, ties to even) is a single rounding: bf16_round must agree bit for bit
    r = np.random.default_rng(29)
    x = np.concatenate([r.standard_normal(20000), r.standard_normal(2000) * 1e-30, r.standard_normal(2000) * 1e30,
                        [0.0, -0.0, 1.0, -1.0, 2.0 ** -130, 3 * 2.0 ** -135]]).astype(np.float32)
    assert np.array_equal(oracle.bf16_round(x.astype(np.float64)), _bf16(x))
    # exact ties between two bf16 values go to the one with an even last bit
    one = 1.0
    assert oracle.bf16_round(one + 2.0 ** -8) == one                       # 1 + half a step: to 1 (even)
    assert oracle.bf16_round(one + 3 * 2.0 ** -8) == one + 2 * 2.0 ** -7   # to 1 + 2 steps (even)
    assert oracle.bf16_round(one + 2.0 ** -8 + 2.0 ** -40) == one + 2.0 ** -7  # above the tie: up
    # a value whose float32 rounding lands on a tie: one rounding from fp64 and the
    # float32-then-bf16 route disagree, and the oracle takes the single rounding
    v = one + 2.0 ** -8 + 2.0 ** -30
    assert oracle.bf16_round(v) == one + 2.0 ** -7 and _bf16(np.float32(v)) == one


def test_stored_forward_and_backward_close_to_exact():
    # the storage rounding moves results by about the bf16 rounding of the rotated rows
    N, T, w = 200, [8, 13, 21, 34, 55, 89], 8
    q, k, v, do = (_bf16(rand((2, N, 64), s)) for s in (25, 26, 27, 28))
    o1, _ = oracle.rope_sparse_forward(q, k, v, T, w, 0.125)
    o2, _ = oracle.rope_sparse_forward(q, k, v, T, w, 0.125, stored=True)
    assert 0 < np.max(np.abs(o1 - o2)) <= 2e-2
    g1 = oracle.rope_sparse_backward(q, k, v, do, T, w, 0.125)
    g2 = oracle.rope_sparse_backward(q, k, v, do, T, w, 0.125, stored=True)
    for a, b in zip(g1, g2):
        assert np.max(np.abs(a - b)) <= 3e-2


# ---- rotary embedding before the learned-alpha variant's interpolated gather ----

def test_rope_frac_integer_targets_equal_static_rope():
    N, w, R = 150, 6, 128
    q, k, v, do = (rand((2, N, 64), s) for s in (30, 31, 32, 33))
    ds = [d for d, _ in oracle.frac_offset_table("fib", 1.0, w, R)]
    T = oracle.offset_table("fib", 1.0, w, R)
    o1, l1 = oracle.rope_frac_forward(q, k, v, ds, w, 0.125)
    o2, l2 = oracle.rope_sparse_forward(q, k, v, T, w, 0.125)
    assert np.max(np.abs(o1 - o2)) <= 1e-12 and np.max(np.abs(l1 - l2)) <= 1e-12
    g1 = oracle.rope_frac_backward(q, k, v, do, ds, w, 0.125)
    g2 = oracle.rope_sparse_backward(q, k, v, do, T, w, 0.125)
    for a, b in zip(g1[:3], g2):
        assert np.max(np.abs(a - b)) <= 1e-12


def _rf_loss(q, k, v, do, alpha, w, R, scale):
    ds = [d for d, _ in oracle.frac_offset_table("fib", alpha, w, R)]
    o, _ = oracle.rope_frac_forward(q, k, v, ds, w, scale)
    return float(np.sum(o * do))


def test_rope_frac_backward_matches_central_differences():
    N, d, w, R, alpha, scale = 22, 8, 2, 32, 1.23, 0.6
    q, k, v, do = (rand((N, d), s) for s in (34, 35, 36, 37))
    tab = oracle.frac_offset_table("fib", alpha, w, R)
    dq, dk, dv, dd = oracle.rope_frac_backward(q, k, v, do, [x for x, _ in tab], w, scale)
    h = 1e-6
    for X, G in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            old = X[idx]
            X[idx] = old + h
            lp = _rf_loss(q, k, v, do, alpha, w, R, scale)
            X[idx] = old - h
            lm = _rf_loss(q, k, v, do, alpha, w, R, scale)
            X[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        assert np.max(np.abs(num - G)) / max(1.0, np.max(np.abs(G))) <= 1e-6
    ga = oracle.frac_alpha_grad(dd, [f for _, f in tab])
    num = (_rf_loss(q, k, v, do, alpha + h, w, R, scale) - _rf_loss(q, k, v, do, alpha - h, w, R, scale)) / (2 * h)
    assert abs(num - ga) <= 1e-6 * max(1.0, abs(ga))
