"""Pins of the oracle's learned-alpha (fractional offset) functions.

The pages fix only that non-integer offsets alpha * f_k read keys and values
linearly interpolated between rows (explainer page "Depth-Staggered Fibonacci
Spacing for Sparse Attention: Static Schedules Beat Learned Dilation and
Extrapolate Where Dense Attention Fails", Portuguese edition, section
"Metodologia / Arquitetura", item "Implementação"). Each check below compares the
oracle with something independent of its code:
  * integer offsets (alpha = 1, the learned variant's starting point): the static
    oracle, itself pinned by brute force and torch;
  * a linear ramp as values and zero queries: interpolation then reproduces the
    exact position i - d, so the output has a closed form;
  * continuity in alpha across integer crossings (a wrong neighbour row or
    swapped weights jumps there);
  * central differences and torch autograd for every gradient, alpha included.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import fsa_ref


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.fixture(scope="module")
def facts(golden_dir):
    with open(os.path.join(golden_dir, "pages_facts.json")) as f:
        return json.load(f)


def entries(base, alpha, w, R):
    return [d for d, _ in oracle.frac_offset_table(base, alpha, w, R)]


def bases(base, alpha, w, R):
    return [f for _, f in oracle.frac_offset_table(base, alpha, w, R)]


# ----------------------------------------------------------------------------
# table
# ----------------------------------------------------------------------------


def test_table_scales_the_printed_list(facts):
    # d_k = alpha * f_k over the printed list, kept at or beyond the window
    fib = [1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 610, 987]
    assert fib[:4] == facts["fib_list_head"] and fib[-1] == facts["fib_list_last"]
    for alpha in (0.5, 0.77, 1.0, 1.3, 1.5):
        tab = oracle.frac_offset_table("fib", alpha, 8, 1024)
        assert [f for _, f in tab] == [f for f in fib if alpha * f >= 8]
        assert all(d == alpha * f for d, f in tab)


@pytest.mark.parametrize("base,alpha,w,R", [("fib", 1.0, 6, 1024), ("fib", 2.0, 3, 300),
                                            ("pow2", 1.0, 4, 1024), ("pow2", 0.5, 2, 1024)])
def test_integer_tables_equal_static_tables(base, alpha, w, R):
    d = entries(base, alpha, w, R)
    assert all(x == int(x) for x in d)
    assert [int(x) for x in d] == oracle.offset_table(base, alpha, w, R)


# ----------------------------------------------------------------------------
# forward
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("base,alpha,w,R,N", [("fib", 1.0, 4, 64, 80), ("pow2", 1.0, 3, 64, 70),
                                              ("fib", 2.0, 2, 40, 90)])
def test_integer_offsets_reduce_to_static_forward(base, alpha, w, R, N):
    q, k, v = (rand((2, N, 8), s) for s in (1, 2, 3))
    o, l = oracle.frac_forward(q, k, v, entries(base, alpha, w, R), w, 0.4)
    os_, ls = oracle.sparse_forward(q, k, v, oracle.offset_table(base, alpha, w, R), w, 0.4)
    assert np.max(np.abs(o - os_)) <= 1e-12
    assert np.max(np.abs(l - ls)) <= 1e-12


@pytest.mark.parametrize("alpha,w", [(1.3, 4), (0.62, 2), (1.5, 6), (0.9, 1)])
def test_ramp_values_give_exact_mean_position(alpha, w):
    # zero queries: uniform weights over the attended columns. Values hold the
    # position j (channel 0) and 1 (channel 1); an interpolated value then holds the
    # real position i - d, so o_i = mean of {i - o : o < w, o <= i} and {i - d : d <= i}.
    N, R = 70, 64
    ds = entries("fib", alpha, w, R)
    q = np.zeros((N, 4))
    k = rand((N, 4), 5)
    v = np.zeros((N, 4))
    v[:, 0] = np.arange(N)
    v[:, 1] = 1.0
    o, lse = oracle.frac_forward(q, k, v, ds, w, 0.5)
    for i in range(N):
        pos = [i - x for x in range(w) if x <= i] + [i - d for d in ds if d <= i]
        assert abs(o[i, 0] - sum(pos) / len(pos)) <= 1e-12
        assert abs(o[i, 1] - 1.0) <= 1e-12
        assert abs(lse[i] - math.log(len(pos))) <= 1e-12


def test_continuity_across_integer_offsets():
    # at alpha = 1 every d_k = f_k is an integer; just below, phi -> 1 and the key
    # must approach row i - f_k from the older side; just above, phi -> 0 from the
    # newer side. Rows i = f_k lose the entry when d_k passes i, so they are skipped;
    # w is no base value, so no entry crosses the threshold d_k >= w.
    N, w, R = 96, 4, 64
    q, k, v = (rand((2, N, 8), s) for s in (6, 7, 8))
    o0, _ = oracle.frac_forward(q, k, v, entries("fib", 1.0, w, R), w, 0.5)
    skip = set(bases("fib", 1.0, w, R))
    rows = [i for i in range(N) if i not in skip]
    for eps in (-1e-9, 1e-9):
        oe, _ = oracle.frac_forward(q, k, v, entries("fib", 1.0 + eps, w, R), w, 0.5)
        assert np.max(np.abs(oe[:, rows] - o0[:, rows])) <= 1e-6


def test_rows_forward_matches_full():
    N = 150
    ds = entries("fib", 1.37, 5, 128)
    q, k, v = (rand((2, N, 8), s) for s in (9, 10, 11))
    o, l = oracle.frac_forward(q, k, v, ds, 5, 0.3)
    rows = np.array([0, 1, 4, 5, 6, 7, 11, 12, 60, 149])
    orow, lrow = oracle.frac_forward_rows(q, k, v, ds, 5, 0.3, rows)
    assert np.max(np.abs(orow - o[:, rows])) <= 1e-13
    assert np.max(np.abs(lrow - l[:, rows])) <= 1e-13


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------


def _loss(q, k, v, do, alpha, w, R, scale):
    o, _ = oracle.frac_forward(q, k, v, entries("fib", alpha, w, R), w, scale)
    return float(np.sum(o * do))


@pytest.mark.parametrize("alpha,w,N", [(1.23, 2, 24), (0.71, 1, 20), (1.5 - 1e-3, 3, 30)])
def test_backward_matches_central_differences(alpha, w, N):
    R, scale, d = 32, 0.6, 4
    q, k, v, do = (rand((N, d), s) for s in (12, 13, 14, 15))
    ds = entries("fib", alpha, w, R)
    # alpha must sit inside a linear piece: no d_k within the step of an integer
    h = 1e-6
    assert all(abs(x - round(x)) > 100 * h * f for x, f in zip(ds, bases("fib", alpha, w, R)))
    dq, dk, dv, dd = oracle.frac_backward(q, k, v, do, ds, w, scale)
    for X, G in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            old = X[idx]
            X[idx] = old + h
            lp = _loss(q, k, v, do, alpha, w, R, scale)
            X[idx] = old - h
            lm = _loss(q, k, v, do, alpha, w, R, scale)
            X[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        assert np.max(np.abs(num - G)) / max(1.0, np.max(np.abs(G))) <= 1e-6
    ga = oracle.frac_alpha_grad(dd, bases("fib", alpha, w, R))
    num = (_loss(q, k, v, do, alpha + h, w, R, scale) - _loss(q, k, v, do, alpha - h, w, R, scale)) / (2 * h)
    assert abs(num - ga) <= 1e-6 * max(1.0, abs(ga))


def _torch_learned_forward(q, k, v, alpha, fs, w, scale):
    """The learned-alpha attention as gathers with torch autograd: the virtual
    position of entry f for query i is p = i - alpha f; its key mixes rows
    floor(p) and floor(p) + 1 by the fractional part of p (the same two rows
    and weights as the interpolation, parametrised by the position)."""
    N, d = q.shape[-2], q.shape[-1]
    i = torch.arange(N, dtype=torch.float64)
    cols_k, cols_v, masks = [], [], []
    for o in range(w):
        j = torch.arange(N) - o
        ok = j >= 0
        jc = j.clamp(min=0)
        cols_k.append(k[..., jc, :])
        cols_v.append(v[..., jc, :])
        masks.append(ok)
    for f in fs:
        pos = i - alpha * f
        ok = pos >= 0
        lo = torch.floor(pos.detach()).long()
        t = pos - lo.to(torch.float64)  # weight of the newer row floor(p) + 1
        lo_c = lo.clamp(0, N - 1)
        hi_c = (lo + 1).clamp(0, N - 1)
        cols_k.append((1 - t)[:, None] * k[..., lo_c, :] + t[:, None] * k[..., hi_c, :])
        cols_v.append((1 - t)[:, None] * v[..., lo_c, :] + t[:, None] * v[..., hi_c, :])
        masks.append(ok)
    K = torch.stack(cols_k, dim=-2)  # [..., N, C, d]
    V = torch.stack(cols_v, dim=-2)
    M = torch.stack(masks, dim=-1)
    S = scale * torch.sum(q[..., :, None, :] * K, dim=-1)
    S = S.masked_fill(~M, float("-inf"))
    P = torch.softmax(S, dim=-1)
    return torch.sum(P[..., None] * V, dim=-2)


@pytest.mark.parametrize("alpha,w,N", [(1.37, 3, 50), (0.58, 2, 45), (1.11, 6, 64)])
def test_backward_matches_torch_autograd(alpha, w, N):
    R, scale = 64, 0.35
    q, k, v, do = (rand((2, N, 8), s) for s in (16, 17, 18, 19))
    tab = oracle.frac_offset_table("fib", alpha, w, R)
    dq, dk, dv, dd = oracle.frac_backward(q, k, v, do, [x for x, _ in tab], w, scale)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    at = torch.tensor(alpha, dtype=torch.float64, requires_grad=True)
    o = _torch_learned_forward(qt, kt, vt, at, [f for _, f in tab], w, scale)
    o0, _ = oracle.frac_forward(q, k, v, [x for x, _ in tab], w, scale)
    assert np.max(np.abs(o.detach().numpy() - o0)) <= 1e-12
    o.backward(torch.from_numpy(do))
    for g, gt in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        assert np.max(np.abs(g - gt.numpy())) <= 1e-11
    ga = oracle.frac_alpha_grad(dd, [f for _, f in tab])
    assert abs(ga - at.grad.item()) <= 1e-10 * max(1.0, abs(ga))


@pytest.mark.parametrize("alpha,w", [(1.3, 4), (1.0, 3), (0.55, 1)])
def test_alpha_gradient_ramp_closed_form(alpha, w):
    # zero queries and ramp values: o_i[0] is the mean position, and moving d_k by
    # one unit moves that entry's value by -1, so
    # d(loss)/d(d_k) = sum over rows with the entry (and the row i - a - 1) of
    # -dout_i[0] / (number of columns of row i).
    N, R = 60, 64
    tab = oracle.frac_offset_table("fib", alpha, w, R)
    ds = [x for x, _ in tab]
    q = np.zeros((N, 4))
    k = rand((N, 4), 20)
    v = np.zeros((N, 4))
    v[:, 0] = np.arange(N)
    do = rand((N, 4), 21)
    _, _, _, dd = oracle.frac_backward(q, k, v, do, ds, w, 0.5)
    for m, d in enumerate(ds):
        a = math.floor(d)
        want = 0.0
        for i in range(N):
            if i >= d and i - a - 1 >= 0:
                cnt = min(w, i + 1) + sum(1 for x in ds if x <= i)
                want -= do[i, 0] / cnt
        assert abs(dd[m] - want) <= 1e-12


def test_rows_backward_matches_full():
    N = 140
    ds = entries("fib", 1.21, 4, 128)
    q, k, v, do = (rand((2, N, 8), s) for s in (22, 23, 24, 25))
    dq, dk, dv, _ = oracle.frac_backward(q, k, v, do, ds, 4, 0.3)
    rows = np.array([0, 1, 3, 4, 5, 9, 10, 30, 100, 139])
    rq, rk, rv = oracle.frac_backward_rows(q, k, v, do, ds, 4, 0.3, rows)
    for a, b in ((rq, dq), (rk, dk), (rv, dv)):
        assert np.max(np.abs(a - b[:, rows])) <= 1e-12


def test_gradient_sums():
    # every softmax row sums to one and the interpolation weights sum to one, so the
    # rows of dV add up to the rows of dO; a constant added to every key leaves the
    # scores' softmax unchanged, so the rows of dK add up to zero
    N = 120
    ds = entries("fib", 0.83, 6, 128)
    q, k, v, do = (rand((N, 8), s) for s in (26, 27, 28, 29))
    _, dk, dv, _ = oracle.frac_backward(q, k, v, do, ds, 6, 0.3)
    assert np.allclose(dv.sum(0), do.sum(0), atol=1e-11)
    assert np.allclose(dk.sum(0), 0.0, atol=1e-11)


# ----------------------------------------------------------------------------
# planted mistakes: the pins above must catch plausible oracle bugs
# ----------------------------------------------------------------------------


def _neighbour_newer(x, d):
    # interpolating toward the newer row i - a + 1 instead of the older row i - a - 1
    N = x.shape[-2]
    a, phi, i0 = fsa_ref._split(d)
    i0 = max(i0, a)
    if i0 >= N:
        return i0, None
    near = x[..., i0 - a : N - a, :]
    if phi == 0.0:
        return i0, near.copy()
    newer = np.concatenate([x[..., i0 - a + 1 : N - a, :], x[..., N - a - 1 : N - a, :]], axis=-2)
    return i0, (1.0 - phi) * near + phi * newer


def _weights_swapped(x, d):
    N = x.shape[-2]
    a, phi, i0 = fsa_ref._split(d)
    if i0 >= N:
        return i0, None
    near = x[..., i0 - a : N - a, :]
    if phi == 0.0:
        return i0, near.copy()
    far = x[..., i0 - a - 1 : N - a - 1, :]
    return i0, phi * near + (1.0 - phi) * far


@pytest.mark.parametrize("bad", [_neighbour_newer, _weights_swapped])
def test_planted_interpolation_mistakes_are_caught(monkeypatch, bad):
    monkeypatch.setattr(fsa_ref, "_virtual_rows", bad)
    N, w, R = 96, 4, 64
    q, k, v = (rand((2, N, 8), s) for s in (6, 7, 8))
    skip = set(bases("fib", 1.0, w, R))
    rows = [i for i in range(N) if i not in skip]
    o0, _ = oracle.frac_forward(q, k, v, entries("fib", 1.0, w, R), w, 0.5)
    oe, _ = oracle.frac_forward(q, k, v, entries("fib", 1.0 - 1e-9, w, R), w, 0.5)
    assert np.max(np.abs(oe[:, rows] - o0[:, rows])) > 1e-3


# ----------------------------------------------------------------------------
# the backward handed its forward outputs (o, lse)
# ----------------------------------------------------------------------------


def _small_case(seed=50, N=90, alpha=1.27, w=5, R=64):
    q, k, v, do = (rand((2, N, 8), seed + s) for s in range(4))
    ds = entries("fib", alpha, w, R)
    return q, k, v, do, ds, w


def test_given_exact_outputs_reproduce_the_backward():
    q, k, v, do, ds, w = _small_case()
    o, lse = oracle.frac_forward(q, k, v, ds, w, 0.4)
    a = oracle.frac_backward(q, k, v, do, ds, w, 0.4)
    b = oracle.frac_backward(q, k, v, do, ds, w, 0.4, o=o, lse=lse)
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) <= 1e-12


def test_given_lse_scales_every_gradient():
    # P = exp(s - lse): adding c to lse multiplies every P and dS, hence every gradient, by exp(-c)
    q, k, v, do, ds, w = _small_case(60)
    o, lse = oracle.frac_forward(q, k, v, ds, w, 0.4)
    a = oracle.frac_backward(q, k, v, do, ds, w, 0.4, o=o, lse=lse)
    b = oracle.frac_backward(q, k, v, do, ds, w, 0.4, o=o, lse=lse + 0.7)
    for x, y in zip(a, b):
        assert np.allclose(y, math.exp(-0.7) * x, rtol=1e-12, atol=1e-13)


def test_given_o_enters_through_d_only_and_affinely():
    # D = <dout, o> enters dS = P (dP - D) linearly: the gradients are affine in o, and move
    q, k, v, do, ds, w = _small_case(70)
    o, lse = oracle.frac_forward(q, k, v, ds, w, 0.4)
    delta = 1e-3 * rand(o.shape, 77)
    g0 = oracle.frac_backward(q, k, v, do, ds, w, 0.4, o=o, lse=lse)
    g1 = oracle.frac_backward(q, k, v, do, ds, w, 0.4, o=o + delta, lse=lse)
    g2 = oracle.frac_backward(q, k, v, do, ds, w, 0.4, o=o + 2 * delta, lse=lse)
    for n, (a, b, c) in enumerate(zip(g0, g1, g2)):
        if n != 2:
            assert np.max(np.abs(b - a)) > 1e-8
        assert np.allclose(c - a, 2 * (b - a), rtol=1e-7, atol=1e-12)
    # dV does not involve D
    assert np.max(np.abs(g1[2] - g0[2])) <= 1e-13
