"""GPU parity of the learned-alpha variant (fractional entries, interpolated K/V
rows) through the C ABI, against the fp64 oracle.

Bars: O, LSE, dQ, dK, dV within max-abs 1e-2 (bf16 inputs, fp32 accumulation);
the table bit-exact in its integer part and base value.

The alpha gradient is a sum over every row of every head, with heavy
cancellation, so its bars are derived from the arithmetic:
  * handed the oracle's own O (rounded to bf16) and LSE (rounded to fp32), the
    backward must reproduce the oracle's backward given those same inputs
    (P = exp(s - lse), D = <dO, O>): every per-row term is fp32 arithmetic on
    exact bf16 products (relative error about 1e-6), summed in fp32 over at most
    64 rows of a tile and in fp64 over tiles, so each entry's derivative must
    agree within 1e-5 of the sum of its terms' absolute values;
  * fed by the GPU forward (end to end), D = <dO, O> uses the forward's bf16 O,
    which differs from the exact O by at most 2^-8 |O| (rounding) plus the
    forward's own 1e-2 bar; through dS = P (dP - D) that moves entry t's
    derivative by at most sum_i scale P_it |s_far - s_near|_it dD_i (entry_bounds):
    a worst-case bound, since the rounding of O is what the exact gradient
    does not see."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from fibonacci_offset_transformer_amd import fsa, schedules, synth

pytestmark = pytest.mark.gpu

TOL = 1e-2


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def inputs(workload, layer, shape, grad=False):
    t = synth.layer_inputs(workload, layer, shape, torch.bfloat16, with_grad=grad)
    return {k: v.to(dev()) for k, v in t.items()}


def check(name, gpu, ref, tol=TOL):
    err = float(np.max(np.abs(synth.as_f64(gpu) - ref))) if ref.size else 0.0
    note(f"  {name}: max|err|={err:.3e} max|ref|={float(np.max(np.abs(ref))) if ref.size else 0:.3f} tol={tol}")
    assert err <= tol, (name, err)


def entry_bounds(q, k, v, do, tab, w, scale):
    """Per-entry error bound of d(loss)/d(d_t) for one head (see the module text)."""
    N = q.shape[0]
    ds = [d for d, _ in tab]
    P, _, _ = oracle.frac_probabilities(q, k, ds, w, scale)
    o, _ = oracle.frac_forward(q, k, v, ds, w, scale)
    D = np.sum(do * o, -1)
    dD = np.sum(np.abs(do) * (2.0 ** -8 * np.abs(o) + 1e-2), -1)
    out = np.zeros(len(tab))
    for m, (d, _) in enumerate(tab):
        a = math.floor(d)
        phi = d - a
        s0 = a + 1  # rows with the entry and the far row
        if s0 >= N:
            continue
        r = np.arange(s0, N)
        kn, kf, vn, vf = k[r - a], k[r - a - 1], v[r - a], v[r - a - 1]
        p = P[r, w + m]
        ds_raw = np.sum(q[r] * (kf - kn), -1)
        ddp = np.sum(do[r] * (vf - vn), -1)
        dS = p * (np.sum(do[r] * ((1 - phi) * vn + phi * vf), -1) - D[r])
        out[m] = (np.sum(scale * p * np.abs(ds_raw) * dD[r])
                  + 1e-3 * np.sum(np.abs(scale * dS * ds_raw) + np.abs(p * ddp)) + 1e-6)
    return out


def frac_fwd_case(workload, B, H, N, base, alpha, w, R, heads=None, layer=0, scale=0.125):
    x = inputs(workload, layer, (B, H, N, 64))
    note(f"frac forward wl={workload} layer={layer} B={B} H={H} N={N} base={base} alpha={alpha} w={w} R={R}")
    kw = dict(alpha=alpha, w=w, R=R, base=base, scale=scale)
    o, lse = fsa.frac_forward(x["q"], x["k"], x["v"], out_dtype=torch.float32, **kw)
    o_lo, lse_lo = fsa.frac_forward(x["q"], x["k"], x["v"], out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_lo, o.to(torch.bfloat16))
    assert torch.equal(lse_lo, lse)
    ds = [d for d, _ in oracle.frac_offset_table(base, alpha, w, R)]
    sel = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in sel:
        q, k, v = (synth.as_f64(x[t][b, h]) for t in ("q", "k", "v"))
        ro, rl = oracle.frac_forward(q, k, v, ds, w, scale)
        check(f"o[{b},{h}]", o[b, h], ro)
        check(f"lse[{b},{h}]", lse[b, h], rl)
    return x, o_lo, lse


def frac_bwd_case(workload, B, H, N, base, alpha, w, R, heads=None, layer=0, scale=0.125, all_heads_alpha=True):
    x = inputs(workload, layer, (B, H, N, 64), grad=True)
    note(f"frac backward wl={workload} layer={layer} B={B} H={H} N={N} base={base} alpha={alpha} w={w} R={R}")
    kw = dict(alpha=alpha, w=w, R=R, base=base, scale=scale)
    o, lse = fsa.frac_forward(x["q"], x["k"], x["v"], **kw)
    g = fsa.frac_backward(x["q"], x["k"], x["v"], o, lse, x["do"], out_dtype=torch.float32, **kw)
    g_lo = fsa.frac_backward(x["q"], x["k"], x["v"], o, lse, x["do"], out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), g_lo[:3], g[:3]):
        assert torch.equal(a, b.to(torch.bfloat16)), name
    assert torch.equal(g_lo[3], g[3]) and torch.equal(g_lo[4], g[4])  # the alpha gradient ignores out_dtype
    tab = oracle.frac_offset_table(base, alpha, w, R)
    ds = [d for d, _ in tab]
    sel = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in sel:
        q, k, v, do = (synth.as_f64(x[t][b, h]) for t in ("q", "k", "v", "do"))
        rq, rk, rv, _ = oracle.frac_backward(q, k, v, do, ds, w, scale)
        check(f"dq[{b},{h}]", g[0][b, h], rq)
        check(f"dk[{b},{h}]", g[1][b, h], rk)
        check(f"dv[{b},{h}]", g[2][b, h], rv)
    if all_heads_alpha:
        dd = np.zeros(len(tab))
        bound = np.zeros(len(tab))
        for b in range(B):
            for h in range(H):
                q, k, v, do = (synth.as_f64(x[t][b, h]) for t in ("q", "k", "v", "do"))
                dd += oracle.frac_backward(q, k, v, do, ds, w, scale)[3]
                bound += entry_bounds(q, k, v, do, tab, w, scale)
        got = synth.as_f64(g[4])
        assert got.shape == dd.shape
        fs = np.array([f for _, f in tab], dtype=np.float64)
        ga = oracle.frac_alpha_grad(dd, fs)
        ga_bound = float(np.sum(fs * bound))
        err_t = np.abs(got - dd)
        ratio = max([float(e / b) for e, b in zip(err_t, bound) if b > 0], default=0.0)
        note(f"  doffs: max|err|/bound={ratio:.3f}")
        assert np.all(err_t <= bound), (err_t, bound)
        err_a = abs(float(g[3].item()) - ga)
        note(f"  dalpha: gpu={float(g[3].item()):.6f} ref={ga:.6f} err={err_a:.3e} bound={ga_bound:.3e}")
        assert err_a <= ga_bound
    return x, g


SMALL = [
    # (N, base, alpha, w, R)
    (1, "fib", 1.3, 16, 256),
    (17, "fib", 1.3, 16, 256),
    (100, "fib", 0.77, 6, 256),
    (300, "fib", 1.3, 16, 256),
    (300, "fib", 0.5 + 1 / 15, 8, 256),
    (300, "fib", 1.5, 12, 256),      # half-integer and integer targets
    (300, "fib", 1.0, 64, 1024),     # integer targets (the learned variant's start)
    (300, "pow2", 1.37, 10, 1024),
    (257, "fib", 1.1, 1, 1024),      # w = 1: every Fibonacci entry, small targets
    (200, "fib", 0.53, 1, 300),      # entries sharing a floor
    (1100, "fib", 1.21, 6, 1024),    # more than eight entries
    (130, "fib", 1.44, 64, 1024),
]


@pytest.mark.parametrize("N,base,alpha,w,R", SMALL)
def test_frac_forward_small(N, base, alpha, w, R):
    frac_fwd_case(40, 2, 2, N, base, alpha, w, R)


@pytest.mark.parametrize("N,base,alpha,w,R", SMALL)
def test_frac_backward_small(N, base, alpha, w, R):
    frac_bwd_case(41, 2, 2, N, base, alpha, w, R)


def test_frac_table_matches_oracle():
    for a in schedules.linear_stagger(16) + [1.0, 0.53, 1.37]:
        got = fsa.frac_offsets(a, 64, 1024)
        want = oracle.frac_offset_table("fib", a, 64, 1024)
        assert [(x, f) for x, _, f in got] == [(math.floor(d), f) for d, f in want]


def test_frac_full_size_stagger_layers():
    # the training-step shape [2, 8, 4096, 64], w = 64, R = 1024, with the stagger
    # schedule's alphas taken as learned values (unrounded targets)
    alphas = schedules.linear_stagger(16)
    rng = np.random.default_rng(42)
    for l in (1, 6, 13):
        b, h = int(rng.integers(0, 2)), int(rng.integers(0, 8))
        frac_fwd_case(42, 2, 8, 4096, "fib", alphas[l], 64, 1024, heads=[(b, h)], layer=l)
    frac_bwd_case(42, 2, 8, 4096, "fib", alphas[6], 64, 1024, heads=[(1, 5)], layer=6)


def test_frac_integer_alpha_matches_static_path():
    # at alpha = 1 every target is an integer: both paths compute the static attention
    x = inputs(43, 0, (2, 4, 1500, 64), grad=True)
    kw = dict(alpha=1.0, w=64, R=1024, scale=0.125)
    of, lf = fsa.frac_forward(x["q"], x["k"], x["v"], out_dtype=torch.float32, **kw)
    os_, ls = fsa.forward(x["q"], x["k"], x["v"], out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    assert float((of - os_).abs().max()) <= 2e-3
    assert float((lf - ls).abs().max()) <= 1e-5


@pytest.mark.parametrize("H", [3, 8], ids=["two_kernels", "one_launch"])
def test_frac_bitwise_deterministic_and_workspace_contents_do_not_matter(H):
    x = inputs(44, 0, (1, H, 999, 64), grad=True)
    kw = dict(alpha=1.17, w=64, R=1024, scale=0.125)
    o, lse = fsa.frac_forward(x["q"], x["k"], x["v"], **kw)
    need = fsa.frac_workspace_bytes(torch.bfloat16, 1, H, 999, alpha=1.17, w=64, R=1024)
    runs = []
    for fill in (0, 0x7FC07FC0, -1):  # zeros, NaN bit patterns, all ones
        ws = torch.full((need // 4 + 77,), fill, dtype=torch.int32, device=dev())
        runs.append(fsa.frac_backward(x["q"], x["k"], x["v"], o, lse, x["do"], ws=ws, out_dtype=torch.float32, **kw))
    o2, lse2 = fsa.frac_forward(x["q"], x["k"], x["v"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for other in runs[1:]:
        for a, b in zip(runs[0], other):
            assert torch.equal(a, b)
    assert bool(torch.isfinite(runs[0][3]).all())


@pytest.mark.parametrize("B,H,N,alpha,w", [(2, 4, 777, 1.3, 64), (1, 8, 300, 1.1, 1), (8, 1, 130, 0.7, 16)])
def test_frac_one_launch_equals_per_head(B, H, N, alpha, w):
    # B * H = 8 runs the dQ and dK/dV work in one launch (the alpha reduction waits for
    # every tile's token, on every XCD); one head at a time runs the two kernels. The
    # gradients agree bit for bit; the alpha gradient is the same fp32 tile partials
    # summed in another order (fp64), so it agrees to fp32 rounding of the per-head sums
    x = inputs(50, 0, (B, H, N, 64), grad=True)
    kw = dict(alpha=alpha, w=w, R=1024, scale=0.125)
    o, lse = fsa.frac_forward(x["q"], x["k"], x["v"], **kw)
    note(f"frac one-launch B={B} H={H} N={N} alpha={alpha} w={w}")
    whole = fsa.frac_backward(x["q"], x["k"], x["v"], o, lse, x["do"], out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    da_sum, da_abs, dd_sum = 0.0, 0.0, None
    for b in range(B):
        for h in range(H):
            one = {t: x[t][b:b + 1, h:h + 1].clone() for t in ("q", "k", "v", "do")}
            ref = fsa.frac_backward(one["q"], one["k"], one["v"], o[b:b + 1, h:h + 1].clone(),
                                    lse[b:b + 1, h:h + 1].clone(), one["do"], out_dtype=torch.float32, **kw)
            torch.cuda.synchronize()
            for name, a, r in zip(("dq", "dk", "dv"), whole[:3], ref[:3]):
                assert torch.equal(a[b, h], r[0, 0]), (name, b, h)
            da_sum += float(ref[3][0])
            da_abs += abs(float(ref[3][0]))
            dd_sum = ref[4].double() if dd_sum is None else dd_sum + ref[4].double()
    assert abs(float(whole[3][0]) - da_sum) <= 1e-6 * da_abs + 1e-6, (float(whole[3][0]), da_sum)
    assert float((whole[4].double() - dd_sum).abs().max()) <= 1e-6 * float(dd_sum.abs().max()) + 1e-6


def test_frac_empty_problem_writes_zero_alpha_gradient():
    d = dev()
    q = torch.empty((0, 2, 64, 64), dtype=torch.bfloat16, device=d)
    lse = torch.empty((0, 2, 64), dtype=torch.float32, device=d)
    dalpha = torch.full((1,), float("nan"), device=d)
    doffs = torch.full((8,), float("nan"), device=d)
    _, _, _, da, do_ = fsa.frac_backward(q, q.clone(), q.clone(), q.clone(), lse, q.clone(), alpha=1.3, w=16, R=256,
                                         dalpha=dalpha, doffs=doffs)
    torch.cuda.synchronize()
    assert float(da.item()) == 0.0
    assert bool((do_ == 0).all())


def entry_l1(q, k, v, do, o_given, tab, w, scale):
    """Per entry: sum over rows of |scale dS ds_raw| + |P ddp| with D from o_given (one head)."""
    N = q.shape[0]
    ds = [d for d, _ in tab]
    P, _, _ = oracle.frac_probabilities(q, k, ds, w, scale)
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


def frac_given_case(workload, B, H, N, base, alpha, w, R, layer=0, scale=0.125):
    """The backward handed the oracle's O (bf16) and LSE (fp32): dQ, dK, dV and the alpha
    gradient against the oracle's backward given the same O and LSE."""
    x = inputs(workload, layer, (B, H, N, 64), grad=True)
    note(f"frac backward, oracle-made O/LSE: wl={workload} B={B} H={H} N={N} base={base} alpha={alpha} w={w} R={R}")
    tab = oracle.frac_offset_table(base, alpha, w, R)
    ds = [d for d, _ in tab]
    o_ref = np.zeros((B, H, N, 64))
    lse_ref = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            q, k, v = (synth.as_f64(x[t][b, h]) for t in ("q", "k", "v"))
            o_ref[b, h], lse_ref[b, h] = oracle.frac_forward(q, k, v, ds, w, scale)
    o_in = torch.from_numpy(o_ref).to(torch.bfloat16)
    lse_in = torch.from_numpy(lse_ref).to(torch.float32)
    g = fsa.frac_backward(x["q"], x["k"], x["v"], o_in.to(dev()), lse_in.to(dev()), x["do"], alpha=alpha, w=w,
                          R=R, base=base, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_g, lse_g = synth.as_f64(o_in), synth.as_f64(lse_in)
    dd = np.zeros(len(tab))
    l1 = np.zeros(len(tab))
    for b in range(B):
        for h in range(H):
            q, k, v, do = (synth.as_f64(x[t][b, h]) for t in ("q", "k", "v", "do"))
            rq, rk, rv, rdd = oracle.frac_backward(q, k, v, do, ds, w, scale, o=o_g[b, h], lse=lse_g[b, h])
            check(f"dq[{b},{h}]", g[0][b, h], rq)
            check(f"dk[{b},{h}]", g[1][b, h], rk)
            check(f"dv[{b},{h}]", g[2][b, h], rv)
            dd += rdd
            l1 += entry_l1(q, k, v, do, o_g[b, h], tab, w, scale)
    tol = 1e-5 * l1 + 1e-6
    got = synth.as_f64(g[4])
    err = np.abs(got - dd)
    note(f"  doffs: max|err|/tol={float(np.max(err / tol)) if len(tab) else 0:.4f}")
    assert np.all(err <= tol), (err, tol)
    fs = np.array([f for _, f in tab], dtype=np.float64)
    ga = oracle.frac_alpha_grad(dd, fs)
    err_a = abs(float(g[3].item()) - ga)
    tol_a = float(np.sum(fs * tol))
    note(f"  dalpha: gpu={float(g[3].item()):.6f} ref={ga:.6f} err={err_a:.3e} tol={tol_a:.3e}")
    assert err_a <= tol_a


@pytest.mark.parametrize("N,base,alpha,w,R", [(300, "fib", 1.3, 16, 256), (257, "fib", 1.1, 1, 1024),
                                              (1100, "fib", 1.21, 6, 1024), (300, "fib", 1.0, 64, 1024),
                                              (200, "fib", 0.53, 1, 300), (300, "pow2", 1.37, 10, 1024)])
def test_frac_alpha_gradient_given_outputs_small(N, base, alpha, w, R):
    frac_given_case(45, 2, 2, N, base, alpha, w, R)


def test_frac_alpha_gradient_given_outputs_full_size():
    frac_given_case(46, 2, 8, 4096, "fib", schedules.linear_stagger(16)[9], 64, 1024, layer=9)


# ---------------------------------------------------------------- decode (inference)

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("alpha,w,R,lens", [(1.3, 64, 1024, [1, 5, 64, 65, 80, 333, 700]),
                                            (0.53, 1, 300, [1, 2, 3, 4, 60, 299]),
                                            (1.0, 16, 256, [1, 17, 200]),
                                            (1.37, 8, 1024, [0, -2, 9999, 11])])
def test_frac_decode_against_oracle(dtype, alpha, w, R, lens):
    """fsa_frac_decode on a ragged batch against the oracle's learned-alpha forward row L - 1
    of each cache (lengths outside [1, Lmax] are clamped)."""
    Lmax, H, scale = 700, 2, 0.125
    B = len(lens)
    t = synth.layer_inputs(47, 0, (B, H, Lmax, 64), dtype, with_grad=True)
    x = {k: v.to(dev()) for k, v in t.items()}
    q = x["do"][:, :, 0, :].contiguous()
    sl = torch.tensor(lens, dtype=torch.int32, device=dev())
    note(f"frac decode {dtype} alpha={alpha} w={w} R={R} lens={lens}")
    o, lse = fsa.decode(q, x["k"], x["v"], sl, alpha=alpha, w=w, R=R, scale=scale, out_dtype=torch.float32,
                        fractional=True)
    o_lo, lse_lo = fsa.decode(q, x["k"], x["v"], sl, alpha=alpha, w=w, R=R, scale=scale, fractional=True)
    torch.cuda.synchronize()
    assert torch.equal(o_lo, o.to(o_lo.dtype)) and torch.equal(lse_lo, lse)
    ds = [d for d, _ in oracle.frac_offset_table("fib", alpha, w, R)]
    tol = 1e-5 if dtype == torch.float32 else TOL
    for b, L in enumerate(lens):
        L = min(max(L, 1), Lmax)
        for h in range(H):
            k, v = (synth.as_f64(x[n][b, h, :L]) for n in ("k", "v"))
            qf = np.zeros_like(k)
            qf[L - 1] = synth.as_f64(q[b, h])
            ro, rl = oracle.frac_forward_rows(qf, k, v, ds, w, scale, [L - 1])
            check(f"decode o[{b},{h}] L={L}", o[b, h][None], ro, tol)
            check(f"decode lse[{b},{h}] L={L}", lse[b, h][None], rl, tol)


def test_frac_decode_matches_frac_forward_last_row():
    x = inputs(48, 0, (1, 4, 999, 64))
    kw = dict(alpha=1.21, w=64, R=1024, scale=0.125)
    o, lse = fsa.frac_forward(x["q"], x["k"], x["v"], out_dtype=torch.float32, **kw)
    sl = torch.tensor([999], dtype=torch.int32, device=dev())
    od, ld = fsa.decode(x["q"][:, :, -1].contiguous(), x["k"], x["v"], sl, out_dtype=torch.float32, fractional=True,
                        **kw)
    torch.cuda.synchronize()
    assert float((od - o[:, :, -1]).abs().max()) <= 2e-3
    assert float((ld - lse[:, :, -1]).abs().max()) <= 1e-5


@pytest.mark.parametrize("H", [3, 4], ids=["two_kernels", "one_launch"])
def test_frac_graph_replays_match_eager(H):
    # forward + backward (with the alpha reduction inside the dK/dV work) and a decode step
    # captured in one HIP graph; every replay, with eager work and a clear in between,
    # reproduces the eager results bit for bit
    x = inputs(49, 0, (2, H, 700, 64), grad=True)
    kw = dict(alpha=1.13, w=64, R=1024, scale=0.125)
    bufs = {n: torch.empty_like(x["q"]) for n in ("o", "dq", "dk", "dv")}
    lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device=dev())
    da = torch.empty(1, dtype=torch.float32, device=dev())
    dd = torch.empty(len(fsa.frac_offsets(1.13, 64, 1024)), dtype=torch.float32, device=dev())  # one per entry
    ws = torch.empty(fsa.frac_workspace_bytes(torch.bfloat16, 2, H, 700, alpha=1.13, w=64, R=1024) // 4 + 1,
                     dtype=torch.int32, device=dev())
    qd = x["q"][:, :, -1].contiguous()
    sl = torch.tensor([700, 333], dtype=torch.int32, device=dev())
    od = torch.empty_like(qd)
    ld = torch.empty(qd.shape[:2], dtype=torch.float32, device=dev())

    def step():
        fsa.frac_forward(x["q"], x["k"], x["v"], out=bufs["o"], lse=lse, **kw)
        fsa.frac_backward(x["q"], x["k"], x["v"], bufs["o"], lse, x["do"], dq=bufs["dq"], dk=bufs["dk"],
                          dv=bufs["dv"], dalpha=da, doffs=dd, ws=ws, **kw)
        fsa.decode(qd, x["k"], x["v"], sl, out=od, lse=ld, fractional=True, **kw)

    outs = dict(bufs, lse=lse, da=da, dd=dd, od=od, ld=ld)
    step()
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in outs.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in outs.values():
            t.zero_()
        fsa.frac_forward(x["k"], x["q"], x["v"], **kw)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in outs:
            assert torch.equal(outs[n], ref[n]), (rep, n)


@pytest.mark.parametrize("H", [3, 8], ids=["two_kernels", "one_launch"])
def test_small_window_backward_with_sharp_attention(H):
    # as the static test of the same name: scale 1/2 at w = 8, where bf16 shares of P and
    # dS would move a gradient by up to about 0.02 and the fp32 shares below w = 64 keep it
    # within 1e-2; the backward is handed the oracle's own O (bf16) and LSE
    B, N, w, alpha, R, scale = 1, 400, 8, 1.3, 1024, 0.5
    x = inputs(42, 0, (B, H, N, 64), grad=True)
    ds = [d for d, _ in oracle.frac_offset_table("fib", alpha, w, R)]
    o_ref, lse_ref = np.zeros((B, H, N, 64)), np.zeros((B, H, N))
    for h in range(H):
        q, k, v = (synth.as_f64(x[t][0, h]) for t in ("q", "k", "v"))
        o_ref[0, h], lse_ref[0, h] = oracle.frac_forward(q, k, v, ds, w, scale)
    o_in = torch.from_numpy(o_ref).to(torch.bfloat16)
    lse_in = torch.from_numpy(lse_ref).to(torch.float32)
    g = fsa.frac_backward(x["q"], x["k"], x["v"], o_in.to(dev()), lse_in.to(dev()), x["do"], alpha=alpha, w=w, R=R,
                          scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    note(f"sharp attention learned-alpha backward B={B} H={H} N={N} w={w} scale={scale}")
    og, lg = synth.as_f64(o_in), synth.as_f64(lse_in)
    for h in range(H):
        q, k, v, do = (synth.as_f64(x[t][0, h]) for t in ("q", "k", "v", "do"))
        ref = oracle.frac_backward(q, k, v, do, ds, w, scale, o=og[0, h], lse=lg[0, h])
        for name, got, want in zip(("dq", "dk", "dv"), g[:3], ref[:3]):
            check(f"{name}[{h}]", got[0, h], want, 1e-2)
