"""Seeded random sweep of small configurations through the C ABI, every head against
the fp64 oracle: the static path (bf16 and fp32, any window), the learned-alpha
variant and the rotary variant (bf16, w <= 64).

Sequence lengths, windows, alphas, reaches and bases are drawn from a fixed seed, so
the sweep covers ragged tails, tables of 0 to 15 entries, windows wider than a tile
and single-row sequences; seeds 40 to 51 draw B * H = 8, whose bf16 backward runs as
one launch. Forward outputs are compared at the usual bars (1e-5 fp32,
1e-2 bf16). The backward is handed the oracle's own O (rounded to the input dtype)
and LSE (rounded to fp32), and compared with the oracle's backward of those same
inputs (P = exp(s - lse), D = <dO, o>); for the learned-alpha variant the alpha
gradient must agree within 1e-5 of the sum of its terms' absolute values (over rotated
rows, plus the allowance of rope_rounding for elements next to a rounding boundary)."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import rope_rounding
from fibonacci_offset_transformer_amd import fsa, synth

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2}


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(name, gpu, ref, tol):
    err = float(np.max(np.abs(synth.as_f64(gpu) - ref))) if ref.size else 0.0
    note(f"  {name}: max|err|={err:.3e} tol={tol}")
    assert err <= tol, (name, err, tol)
    return err


def draw(seed, wide_windows, heads8=False):
    r = np.random.default_rng(seed)
    N = int(r.choice([1, 2, 63, 64, 65, int(r.integers(3, 400)), int(r.integers(400, 1500))]))
    w = int(r.integers(1, 130 if wide_windows else 65))
    alpha = float(r.uniform(0.5, 1.5))
    R = int(r.choice([1, 2, 64, 200, 1024, 2048]))
    base = "pow2" if r.random() < 0.3 else "fib"
    B, H = int(r.integers(1, 3)), int(r.integers(1, 3))
    if heads8:  # B * H = 8 with sparse offsets below N: the backward runs as one launch
        B, H = [(1, 8), (2, 4), (4, 2), (8, 1)][int(r.integers(0, 4))]
        N = int(r.choice([65, 130, 257, int(r.integers(66, 700))]))
        R = int(r.choice([64, 200, 1024, 2048]))
    return B, H, N, w, alpha, R, base


def oracle_outputs(x, B, H, fwd):
    o = np.zeros(tuple(x["q"].shape))
    lse = np.zeros(tuple(x["q"].shape[:3]))
    for b in range(B):
        for h in range(H):
            q, k, v = (synth.as_f64(x[t][b, h]) for t in ("q", "k", "v"))
            o[b, h], lse[b, h] = fwd(q, k, v)
    return o, lse


STATIC = [(s, dt) for s in range(12) for dt in (torch.float32, torch.bfloat16)]
ONE_LAUNCH = [(s, torch.bfloat16) for s in range(40, 52)]


@pytest.mark.parametrize("seed,dtype", STATIC + ONE_LAUNCH,
                         ids=[f"{s}-{'f32' if d == torch.float32 else 'bf16'}" for s, d in STATIC + ONE_LAUNCH])
def test_sweep_static(seed, dtype):
    static_case(seed, dtype, wide_windows=seed < 40, heads8=seed >= 40)


# Narrow windows (w <= 5) drawn the same way, where a query's one to five keys each carry
# a large share of its probability. On these draws a single bf16 rounding of each sparse
# pair's P and dS moves some gradient by 1.0e-2 to 1.4e-2 (a CPU search over seeds 0-4499
# with that one rounding put into the oracle's backward); the window backward carries
# those weights as fp32 words for windows below 64, and these cases pin it. heads8 draws
# B * H = 8 (one-launch backward), the others the two-kernel backward.
SMALL_WINDOW = [(1332, True), (3675, True), (2437, True), (3120, True), (2477, True), (2591, True),
                (1864, True), (547, True), (2723, True), (2834, True), (4180, True), (419, True),
                (1332, False), (737, False), (885, False), (1864, False)]


@pytest.mark.parametrize("seed,heads8", SMALL_WINDOW, ids=[f"{s}-{'one' if h else 'two'}" for s, h in SMALL_WINDOW])
def test_small_window_backward(seed, heads8):
    B, H, N, w, alpha, R, base = draw(100 + seed, wide_windows=False, heads8=heads8)
    assert w <= 5 and (B * H == 8) == heads8
    static_case(seed, torch.bfloat16, wide_windows=False, heads8=heads8)


def static_case(seed, dtype, wide_windows, heads8):
    B, H, N, w, alpha, R, base = draw(100 + seed, wide_windows=wide_windows, heads8=heads8)
    note(f"static {dtype} seed={seed} B={B} H={H} N={N} w={w} alpha={alpha:.4f} R={R} base={base}")
    x = {k: v.to(dev()) for k, v in synth.layer_inputs(80 + seed, 0, (B, H, N, 64), dtype, with_grad=True).items()}
    kw = dict(alpha=alpha, w=w, R=R, base=base, scale=0.125)
    T = oracle.offset_table(base, alpha, w, R)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], out_dtype=torch.float32, **kw)
    ro, rl = oracle_outputs(x, B, H, lambda q, k, v: oracle.sparse_forward(q, k, v, T, w, 0.125))
    torch.cuda.synchronize()
    check("o", o, ro, TOL[dtype])
    check("lse", lse, rl, TOL[dtype])
    o_in = torch.from_numpy(ro).to(dtype)
    lse_in = torch.from_numpy(rl).to(torch.float32)
    g = fsa.backward(x["q"], x["k"], x["v"], o_in.to(dev()), lse_in.to(dev()), x["do"], out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    og, lg = synth.as_f64(o_in), synth.as_f64(lse_in)
    for b in range(B):
        for h in range(H):
            q, k, v, do = (synth.as_f64(x[t][b, h]) for t in ("q", "k", "v", "do"))
            ref = oracle.sparse_backward(q, k, v, do, T, w, 0.125, o=og[b, h], lse=lg[b, h])
            for name, got, want in zip(("dq", "dk", "dv"), g, ref):
                check(f"{name}[{b},{h}]", got[b, h], want, TOL[dtype])


def _entry_l1(q, k, v, do, o_given, tab, w, scale):
    N = q.shape[0]
    P, _, _ = oracle.frac_probabilities(q, k, [d for d, _ in tab], w, scale)
    D = np.sum(do * o_given, -1)
    out = np.zeros(len(tab))
    for m, (d, _) in enumerate(tab):
        a = math.floor(d)
        phi = d - a
        if a + 1 >= N:
            continue
        r = np.arange(a + 1, N)
        kn, kf, vn, vf = k[r - a], k[r - a - 1], v[r - a], v[r - a - 1]
        p = P[r, w + m]
        ds_raw = np.sum(q[r] * (kf - kn), -1)
        dS = p * (np.sum(do[r] * ((1 - phi) * vn + phi * vf), -1) - D[r])
        out[m] = np.sum(np.abs(scale * dS * ds_raw) + np.abs(p * np.sum(do[r] * (vf - vn), -1)))
    return out


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("rope", [False, True], ids=["plain", "rope"])
def test_sweep_learned_alpha(seed, rope):
    B, H, N, w, alpha, R, base = draw(200 + seed, wide_windows=False)
    note(f"learned alpha rope={rope} B={B} H={H} N={N} w={w} alpha={alpha:.4f} R={R} base={base}")
    x = {k: v.to(dev()) for k, v in synth.layer_inputs(90 + seed, 0, (B, H, N, 64), torch.bfloat16,
                                                      with_grad=True).items()}
    kw = dict(alpha=alpha, w=w, R=R, base=base, scale=0.125)
    tab = oracle.frac_offset_table(base, alpha, w, R)
    ds = [d for d, _ in tab]
    if rope:
        table = fsa.rope_table(N, device=dev())
        o, lse = fsa.rope_frac_forward(x["q"], x["k"], x["v"], table, out_dtype=torch.float32, **kw)
        rot = oracle.rope_store_bf16
        fwd_ref = lambda q, k, v: oracle.rope_frac_forward(q, k, v, ds, w, 0.125, stored=True)
    else:
        o, lse = fsa.frac_forward(x["q"], x["k"], x["v"], out_dtype=torch.float32, **kw)
        rot = lambda a: a
        fwd_ref = lambda q, k, v: oracle.frac_forward(q, k, v, ds, w, 0.125)
    ro, rl = oracle_outputs(x, B, H, fwd_ref)
    torch.cuda.synchronize()
    check("o", o, ro, 1e-2)
    check("lse", lse, rl, 1e-2)
    o_in = torch.from_numpy(ro).to(torch.bfloat16)
    lse_in = torch.from_numpy(rl).to(torch.float32)
    if rope:
        g = fsa.rope_frac_backward(x["q"], x["k"], x["v"], table, o_in.to(dev()), lse_in.to(dev()), x["do"],
                                   out_dtype=torch.float32, **kw)
    else:
        g = fsa.frac_backward(x["q"], x["k"], x["v"], o_in.to(dev()), lse_in.to(dev()), x["do"],
                              out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    og, lg = synth.as_f64(o_in), synth.as_f64(lse_in)
    dd = np.zeros(len(tab))
    l1 = np.zeros(len(tab))
    allow = np.zeros(len(tab))
    for b in range(B):
        for h in range(H):
            q, k, v, do = (synth.as_f64(x[t][b, h]) for t in ("q", "k", "v", "do"))
            if rope:
                ref = oracle.rope_frac_backward(q, k, v, do, ds, w, 0.125, stored=True, o=og[b, h], lse=lg[b, h])
            else:
                ref = oracle.frac_backward(q, k, v, do, ds, w, 0.125, o=og[b, h], lse=lg[b, h])
            for name, got, want in zip(("dq", "dk", "dv"), g[:3], ref[:3]):
                check(f"{name}[{b},{h}]", got[b, h], want, 1e-2)
            dd += ref[3]
            l1 += _entry_l1(rot(q), rot(k), v, do, og[b, h], tab, w, 0.125)
            if rope:  # rotated elements next to a bf16 rounding boundary may hold either neighbour
                allow += rope_rounding.entry_grad_allowance(q, k, v, do, ds, w, 0.125, og[b, h], lg[b, h])[0]
    tol = 1e-5 * l1 + 1e-6 + allow
    got = synth.as_f64(g[4])
    assert np.all(np.abs(got - dd) <= tol), (got, dd, tol)
    fs = np.array([f for _, f in tab], dtype=np.float64)
    assert abs(float(g[3].item()) - oracle.frac_alpha_grad(dd, fs)) <= float(np.sum(fs * tol))


@pytest.mark.parametrize("seed", range(12))
def test_sweep_rope_static(seed):
    B, H, N, w, alpha, R, base = draw(300 + seed, wide_windows=False)
    note(f"rope B={B} H={H} N={N} w={w} alpha={alpha:.4f} R={R} base={base}")
    x = {k: v.to(dev()) for k, v in synth.layer_inputs(110 + seed, 0, (B, H, N, 64), torch.bfloat16,
                                                      with_grad=True).items()}
    kw = dict(alpha=alpha, w=w, R=R, base=base, scale=0.125)
    table = fsa.rope_table(N + 7, device=dev())
    T = oracle.offset_table(base, alpha, w, R)
    o, lse = fsa.rope_forward(x["q"], x["k"], x["v"], table, out_dtype=torch.float32, **kw)
    ro, rl = oracle_outputs(x, B, H, lambda q, k, v: oracle.rope_sparse_forward(q, k, v, T, w, 0.125, stored=True))
    torch.cuda.synchronize()
    check("o", o, ro, 1e-2)
    check("lse", lse, rl, 1e-2)
    o_in = torch.from_numpy(ro).to(torch.bfloat16)
    lse_in = torch.from_numpy(rl).to(torch.float32)
    g = fsa.rope_backward(x["q"], x["k"], x["v"], table, o_in.to(dev()), lse_in.to(dev()), x["do"],
                          out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    og, lg = synth.as_f64(o_in), synth.as_f64(lse_in)
    for b in range(B):
        for h in range(H):
            q, k, v, do = (synth.as_f64(x[t][b, h]) for t in ("q", "k", "v", "do"))
            ref = oracle.rope_sparse_backward(q, k, v, do, T, w, 0.125, stored=True, o=og[b, h], lse=lg[b, h])
            for name, got, want in zip(("dq", "dk", "dv"), g, ref):
                check(f"{name}[{b},{h}]", got[b, h], want, 1e-2)
