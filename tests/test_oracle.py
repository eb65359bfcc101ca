"""Pins of the fp64 oracle against what the pages and mathematics fix.

None of these checks re-types the oracle's own formula: each compares it with
something independent of it (a value printed on the pages, a closed form, a
library routine, a brute-force N x N evaluation, finite differences, torch
autograd) so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them. The planted-mistake tests at
the end show that for a few such mistakes.
"""
import decimal
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import fsa_ref

# ----------------------------------------------------------------------------
# helpers that do NOT use the oracle's code
# ----------------------------------------------------------------------------


def binet(n):
    """n-th Fibonacci number (F(1)=F(2)=1) from the closed form round(phi^n/sqrt5)."""
    phi = (1.0 + math.sqrt(5.0)) / 2.0
    return int(round(phi ** n / math.sqrt(5.0)))


def independent_table(base, alpha, w, R, rounding="even"):
    """Offset table via the closed form for the base and the language's rounding."""
    if base == "fib":
        vals, n = [], 2          # distinct values start at F(2) = 1, F(3) = 2
        while binet(n) < R:
            vals.append(binet(n))
            n += 1
    else:
        vals = [1 << k for k in range(0, 64) if (1 << k) < R]
    if rounding == "even":
        sc = [round(alpha * f) for f in vals]      # Python round(): ties to even
    else:
        sc = [int(decimal.Decimal(alpha * f).quantize(decimal.Decimal(1),
                                                     rounding=decimal.ROUND_HALF_UP))
              for f in vals]
    return sorted({o for o in sc if o >= w})


def brute_mask(N, T, w):
    """N x N boolean mask, True where query i attends key j."""
    offs = set(range(w)) | set(T)
    M = np.zeros((N, N), dtype=bool)
    for i in range(N):
        for j in range(N):
            M[i, j] = (j <= i) and ((i - j) in offs)
    return M


def brute_attention(q, k, v, M, scale):
    """Full-matrix masked softmax attention with one head: returns o, lse."""
    S = scale * (q @ k.T)
    S = np.where(M, S, -np.inf)
    mx = S.max(axis=1, keepdims=True)
    e = np.exp(S - mx)
    l = e.sum(axis=1, keepdims=True)
    return (e / l) @ v, (mx + np.log(l))[:, 0]


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.fixture(scope="module")
def facts(golden_dir):
    with open(os.path.join(golden_dir, "pages_facts.json")) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# offset tables
# ----------------------------------------------------------------------------


def test_fib_list_matches_printed_values(facts):
    # R = 1024 is the reading (training length); the pages print the head and the last value.
    fs = oracle.fibonacci_base(1024)
    assert fs[: len(facts["fib_prefix"])] == facts["fib_prefix"]
    assert fs[: len(facts["fib_list_head"])] == facts["fib_list_head"]
    assert fs[-1] == facts["fib_list_last"]
    assert len(fs) == len(set(fs))  # no repeated 1


@pytest.mark.parametrize("R", [1, 2, 3, 4, 100, 256, 987, 988, 1024, 4096, 1 << 20])
def test_fib_base_matches_binet(R):
    expected, n = [], 2
    while binet(n) < R:
        expected.append(binet(n))
        n += 1
    assert oracle.fibonacci_base(R) == expected


@pytest.mark.parametrize("R", [1, 2, 3, 64, 65, 1024, 1025])
def test_pow2_base_matches_shifts(R):
    assert oracle.pow2_base(R) == [1 << k for k in range(40) if (1 << k) < R]


def test_alpha_one_w1_reproduces_fibonacci():
    # spec check: alpha = 1 with no window absorption gives 1, 2, 3, 5, 8, 13, ...
    assert oracle.offset_table("fib", 1.0, 1, 1024)[:6] == [1, 2, 3, 5, 8, 13]


def test_round_half_even_matches_python_round():
    rng = np.random.default_rng(7)
    xs = [i / 2 for i in range(0, 4000)]  # every tie up to 2000
    xs += list(rng.uniform(0, 3000, 20000))
    xs += [0.5 * f for f in oracle.fibonacci_base(1 << 20)]
    for x in xs:
        assert oracle.round_half_even(float(x)) == round(float(x)), x


def test_round_half_away_matches_decimal():
    xs = [i / 2 for i in range(0, 4000)] + list(np.random.default_rng(8).uniform(0, 3000, 5000))
    for x in xs:
        ref = int(decimal.Decimal(float(x)).quantize(decimal.Decimal(1), rounding=decimal.ROUND_HALF_UP))
        assert oracle.round_half_away(float(x)) == ref, x


def _sweep_alphas():
    al = [0.5 + l / 15.0 for l in range(16)] + [0.5, 1.0, 1.5]
    al += list(np.random.default_rng(11).uniform(0.5, 1.5, 200))
    return al


@pytest.mark.parametrize("base", ["fib", "pow2"])
@pytest.mark.parametrize("rounding", ["even", "away"])
def test_tables_match_independent_construction(base, rounding):
    for alpha in _sweep_alphas():
        for w in (1, 6, 8, 10, 12, 16, 64):
            for R in (1, 2, 256, 1024, 4096):
                got = oracle.offset_table(base, float(alpha), w, R, rounding=rounding)
                assert got == independent_table(base, float(alpha), w, R, rounding), (alpha, w, R)


def test_tables_read_off_the_printed_list():
    # alpha = 1: the entries of the printed list 1..987 that are >= w
    assert oracle.offset_table("fib", 1.0, 64, 1024) == [89, 144, 233, 377, 610, 987]
    assert oracle.offset_table("fib", 1.0, 16, 256) == [21, 34, 55, 89, 144, 233]
    # power-of-2 control reach-matched at R = 1024 with the 64 window
    assert oracle.offset_table("pow2", 1.0, 64, 1024) == [64, 128, 256, 512]


def test_stagger_schedule_endpoints(facts):
    L = facts["n_layers"]
    assert oracle.stagger_alpha(0, L) == facts["stagger_alpha_layer0"]
    assert oracle.stagger_alpha(L - 1, L) == facts["stagger_alpha_layer15"]
    steps = np.diff([oracle.stagger_alpha(l, L) for l in range(L)])
    assert np.allclose(steps, 1.0 / 15.0, rtol=0, atol=1e-15)
    lo, hi = facts["alpha_range"]
    assert all(lo <= oracle.stagger_alpha(l, L) <= hi for l in range(L))


def test_coprime_map_is_a_permutation_and_involution(facts):
    L, c = facts["n_layers"], facts["coprime_step"]
    perm = [oracle.coprime_layer(l, L) for l in range(L)]
    assert sorted(perm) == list(range(L))
    assert all(oracle.coprime_layer(perm[l], L) == l for l in range(L))  # 7*7 = 49 = 1 mod 16
    assert perm == [(c * l) % L for l in range(L)]


def test_rounding_reading_changes_only_tie_layers():
    # At w = 64 and R = 1024 only the alpha = 0.5 and alpha = 1.5 layers have ties that survive.
    changed = [l for l in range(16)
               if oracle.offset_table("fib", oracle.stagger_alpha(l), 64, 1024, "even")
               != oracle.offset_table("fib", oracle.stagger_alpha(l), 64, 1024, "away")]
    assert changed == [0, 15]


# ----------------------------------------------------------------------------
# forward
# ----------------------------------------------------------------------------

CASES = [
    # (N, d, T, w)
    (1, 4, [], 1),
    (5, 3, [], 1),
    (17, 8, [3, 5, 8, 13], 2),
    (33, 8, oracle.offset_table("fib", 1.0, 6, 64), 6),
    (64, 8, oracle.offset_table("fib", 0.5, 8, 64), 8),
    (64, 4, oracle.offset_table("fib", 1.5, 12, 64), 12),
    (40, 8, oracle.offset_table("pow2", 1.0, 4, 64), 4),
    (29, 5, [7, 30, 31], 3),      # offsets reaching past the sequence
]


@pytest.mark.parametrize("N,d,T,w", CASES)
def test_forward_matches_bruteforce_mask(N, d, T, w):
    q, k, v = rand((N, d), 1), rand((N, d), 2), rand((N, d), 3)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.sparse_forward(q, k, v, T, w, scale)
    ob, lb = brute_attention(q, k, v, brute_mask(N, T, w), scale)
    assert np.max(np.abs(o - ob)) <= 1e-12
    assert np.max(np.abs(lse - lb)) <= 1e-12


@pytest.mark.parametrize("N,d,T,w", CASES)
def test_forward_matches_torch_sdpa(N, d, T, w):
    B, H = 2, 3
    q, k, v = rand((B, H, N, d), 4), rand((B, H, N, d), 5), rand((B, H, N, d), 6)
    scale = 1 / math.sqrt(d)
    o, _ = oracle.sparse_forward(q, k, v, T, w, scale)
    M = torch.from_numpy(brute_mask(N, T, w))
    ot = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=M, scale=scale)
    assert np.max(np.abs(o - ot.numpy())) <= 1e-12


def test_rows_sum_to_one():
    q, k = rand((2, 2, 300, 16), 9), rand((2, 2, 300, 16), 10)
    T = oracle.offset_table("fib", 1.0, 16, 256)
    offs, P, _, _ = oracle.sparse_probabilities(q, k, T, 16, 0.25)
    assert np.max(np.abs(P.sum(-1) - 1.0)) <= 1e-14
    # masked entries are exactly zero, and row 0 attends only itself
    assert np.all(P[..., 0, 1:] == 0) and np.all(P[..., 0, 0] == 1)


def test_window_at_least_N_equals_dense_causal():
    N, d = 50, 8
    q, k, v = rand((1, 2, N, d), 12), rand((1, 2, N, d), 13), rand((1, 2, N, d), 14)
    o, lse = oracle.sparse_forward(q, k, v, [], N, 0.3)
    od, ld = oracle.dense_forward(q, k, v, 0.3)
    ot = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True, scale=0.3)
    assert np.max(np.abs(o - ot.numpy())) <= 1e-12
    assert np.max(np.abs(od - ot.numpy())) <= 1e-12
    assert np.max(np.abs(lse - ld)) <= 1e-12


def test_dense_rows_match_dense():
    N, d = 70, 8
    q, k, v = rand((2, N, d), 15), rand((2, N, d), 16), rand((2, N, d), 17)
    od, ld = oracle.dense_forward(q, k, v, 0.2)
    rows = np.array([0, 1, 33, 69])
    orow, lrow = oracle.dense_forward_rows(q, k, v, 0.2, rows)
    assert np.max(np.abs(orow - od[..., rows, :])) <= 1e-13
    assert np.max(np.abs(lrow - ld[..., rows])) <= 1e-13


def test_w1_empty_table_is_identity_on_v():
    N, d = 20, 8
    q, k, v = rand((N, d), 18), rand((N, d), 19), rand((N, d), 20)
    o, lse = oracle.sparse_forward(q, k, v, [], 1, 0.125)
    assert np.array_equal(o, v)
    assert np.allclose(lse, 0.125 * np.einsum("nd,nd->n", q, k), rtol=0, atol=1e-14)


def test_single_row_sequence():
    q, k, v = rand((1, 8), 21), rand((1, 8), 22), rand((1, 8), 23)
    o, _ = oracle.sparse_forward(q, k, v, [89, 144], 64, 0.125)
    assert np.array_equal(o, v)


def test_prefix_consistency():
    # rows of a long run equal a run on the prefix (causality; the 1024 -> 4096 protocol)
    N, Np, d = 400, 150, 8
    T = oracle.offset_table("fib", 1.0, 8, 256)
    q, k, v = rand((2, N, d), 24), rand((2, N, d), 25), rand((2, N, d), 26)
    o, l = oracle.sparse_forward(q, k, v, T, 8, 0.3)
    op, lp = oracle.sparse_forward(q[:, :Np], k[:, :Np], v[:, :Np], T, 8, 0.3)
    assert np.max(np.abs(o[:, :Np] - op)) <= 1e-14
    assert np.max(np.abs(l[:, :Np] - lp)) <= 1e-14


def test_forward_rows_match_full():
    N, d = 300, 8
    T = oracle.offset_table("fib", 1.0, 16, 256)
    q, k, v = rand((2, N, d), 27), rand((2, N, d), 28), rand((2, N, d), 29)
    o, l = oracle.sparse_forward(q, k, v, T, 16, 0.3)
    rows = np.array([0, 1, 15, 16, 20, 21, 100, 233, 234, 299])
    orow, lrow = oracle.sparse_forward_rows(q, k, v, T, 16, 0.3, rows)
    assert np.max(np.abs(orow - o[:, rows])) <= 1e-13
    assert np.max(np.abs(lrow - l[:, rows])) <= 1e-13


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------


def _loss(q, k, v, do, T, w, scale):
    o, _ = oracle.sparse_forward(q, k, v, T, w, scale)
    return float(np.sum(o * do))


@pytest.mark.parametrize("N,d,T,w", [(12, 4, [3, 5, 8], 2), (9, 3, [], 9), (10, 4, [4, 6, 7, 20], 1)])
def test_backward_matches_central_differences(N, d, T, w):
    q, k, v, do = rand((N, d), 30), rand((N, d), 31), rand((N, d), 32), rand((N, d), 33)
    scale = 0.7
    dq, dk, dv = oracle.sparse_backward(q, k, v, do, T, w, scale)
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
        rel = np.max(np.abs(num - G)) / max(1.0, np.max(np.abs(G)))
        assert rel <= 1e-6


@pytest.mark.parametrize("N,d,T,w", CASES[2:])
def test_backward_matches_torch_autograd_dense_masked(N, d, T, w):
    B, H = 1, 2
    q, k, v, do = (rand((B, H, N, d), s) for s in (34, 35, 36, 37))
    scale = 1 / math.sqrt(d)
    dq, dk, dv = oracle.sparse_backward(q, k, v, do, T, w, scale)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    M = torch.from_numpy(brute_mask(N, T, w))
    S = scale * (qt @ kt.transpose(-1, -2))
    S = S.masked_fill(~M, float("-inf"))
    o = torch.softmax(S, dim=-1) @ vt
    o.backward(torch.from_numpy(do))
    for g, gt in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        assert np.max(np.abs(g - gt.numpy())) <= 1e-12


def test_backward_rows_match_full():
    N, d = 260, 8
    T = oracle.offset_table("fib", 1.0, 16, 256)
    q, k, v, do = (rand((2, N, d), s) for s in (38, 39, 40, 41))
    dq, dk, dv = oracle.sparse_backward(q, k, v, do, T, 16, 0.3)
    rows = np.array([0, 1, 15, 16, 20, 100, 233, 259])
    rq, rk, rv = oracle.sparse_backward_rows(q, k, v, do, T, 16, 0.3, rows)
    for a, b in ((rq, dq), (rk, dk), (rv, dv)):
        assert np.max(np.abs(a - b[:, rows])) <= 1e-12


def test_gradient_sums():
    # each softmax row sums to 1, so the rows of dV add up to the rows of dO
    N, d = 128, 8
    T = oracle.offset_table("fib", 1.0, 8, 128)
    q, k, v, do = (rand((N, d), s) for s in (42, 43, 44, 45))
    dq, dk, dv = oracle.sparse_backward(q, k, v, do, T, 8, 0.3)
    assert np.allclose(dv.sum(0), do.sum(0), atol=1e-11)
    # adding a constant vector c to every key shifts each row's scores by scale*<q_i,c>,
    # which softmax ignores, so sum_j dK_j = 0
    assert np.allclose(dk.sum(0), 0.0, atol=1e-11)


# ----------------------------------------------------------------------------
# planted mistakes: each pin above must catch a plausible oracle bug
# ----------------------------------------------------------------------------


def _bad_scores_dropped_scale(q, k, offs, scale):
    return fsa_ref.__dict__["_orig_scores"](q, k, offs, 1.0)


def _bad_scores_off_by_one(q, k, offs, scale):
    return fsa_ref.__dict__["_orig_scores"](q, k, [o + 1 if o > 0 else o for o in offs], scale)


def _bad_scores_transposed(q, k, offs, scale):
    return fsa_ref.__dict__["_orig_scores"](k, q, offs, scale)


@pytest.mark.parametrize("bad", [_bad_scores_dropped_scale, _bad_scores_off_by_one, _bad_scores_transposed])
def test_planted_forward_mistakes_are_caught(monkeypatch, bad):
    monkeypatch.setitem(fsa_ref.__dict__, "_orig_scores", fsa_ref._scores)
    monkeypatch.setattr(fsa_ref, "_scores", bad)
    N, d, T, w = 33, 8, [8, 13, 21], 3
    q, k, v = rand((N, d), 1), rand((N, d), 2), rand((N, d), 3)
    o, _ = oracle.sparse_forward(q, k, v, T, w, 0.35)
    ob, _ = brute_attention(q, k, v, brute_mask(N, T, w), 0.35)
    assert np.max(np.abs(o - ob)) > 1e-6


def test_planted_backward_mistake_is_caught(monkeypatch):
    # drop the D term of dS = P (dP - D)
    orig = fsa_ref.sparse_forward

    def zero_o(*a, **kw):
        o, l = orig(*a, **kw)
        return np.zeros_like(o), l

    N, d, T, w = 12, 4, [3, 5, 8], 2
    q, k, v, do = rand((N, d), 30), rand((N, d), 31), rand((N, d), 32), rand((N, d), 33)
    good = oracle.sparse_backward(q, k, v, do, T, w, 0.7)
    monkeypatch.setattr(fsa_ref, "sparse_forward", zero_o)
    bad = fsa_ref.sparse_backward(q, k, v, do, T, w, 0.7)
    monkeypatch.undo()
    # the finite-difference pin sees the good one and rejects the bad one
    h = 1e-6
    idx = (5, 1)
    qp, qm = q.copy(), q.copy()
    qp[idx] += h
    qm[idx] -= h
    num = (_loss(qp, k, v, do, T, w, 0.7) - _loss(qm, k, v, do, T, w, 0.7)) / (2 * h)
    assert abs(num - good[0][idx]) <= 1e-6
    assert abs(num - bad[0][idx]) > 1e-4


def test_planted_rounding_mistake_is_caught():
    # a table built with floor instead of rounding differs from the closed-form construction
    for l in range(16):
        a = oracle.stagger_alpha(l)
        floor_table = sorted({int(math.floor(a * f)) for f in oracle.fibonacci_base(1024)
                              if int(math.floor(a * f)) >= 64})
        if floor_table != independent_table("fib", a, 64, 1024):
            return
    pytest.fail("floor rounding was never distinguished")


# ----------------------------------------------------------------------------
# the backward handed its forward outputs (o, lse)
# ----------------------------------------------------------------------------


def test_given_exact_outputs_reproduce_the_backward():
    N, d, T, w = 90, 8, [8, 13, 21, 34], 5
    q, k, v, do = (rand((2, N, d), s) for s in (80, 81, 82, 83))
    o, lse = oracle.sparse_forward(q, k, v, T, w, 0.4)
    a = oracle.sparse_backward(q, k, v, do, T, w, 0.4)
    b = oracle.sparse_backward(q, k, v, do, T, w, 0.4, o=o, lse=lse)
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) <= 1e-12


def test_given_lse_scales_every_gradient():
    # P = exp(s - lse): adding c to lse multiplies every P and dS, hence every gradient, by exp(-c)
    N, d, T, w = 70, 8, [8, 13, 21], 4
    q, k, v, do = (rand((2, N, d), s) for s in (84, 85, 86, 87))
    o, lse = oracle.sparse_forward(q, k, v, T, w, 0.4)
    a = oracle.sparse_backward(q, k, v, do, T, w, 0.4, o=o, lse=lse)
    b = oracle.sparse_backward(q, k, v, do, T, w, 0.4, o=o, lse=lse - 0.3)
    for x, y in zip(a, b):
        assert np.allclose(y, math.exp(0.3) * x, rtol=1e-12, atol=1e-13)


def test_given_o_enters_through_d_only_and_affinely():
    N, d, T, w = 70, 8, [8, 13, 21], 4
    q, k, v, do = (rand((2, N, d), s) for s in (88, 89, 90, 91))
    o, lse = oracle.sparse_forward(q, k, v, T, w, 0.4)
    delta = 1e-3 * rand(o.shape, 92)
    g0, g1, g2 = (oracle.sparse_backward(q, k, v, do, T, w, 0.4, o=o + c * delta, lse=lse) for c in (0, 1, 2))
    for n, (a, b, c) in enumerate(zip(g0, g1, g2)):
        if n != 2:
            assert np.max(np.abs(b - a)) > 1e-8
        assert np.allclose(c - a, 2 * (b - a), rtol=1e-7, atol=1e-12)
    assert np.max(np.abs(g1[2] - g0[2])) <= 1e-13  # dV does not involve D
