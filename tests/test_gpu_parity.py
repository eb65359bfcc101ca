"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars: offset tables bit-exact; outputs within max-abs 1e-5 for float32 inputs
and 1e-2 for bfloat16 inputs (fp32 accumulation), the tolerances the method's
build target states. Small cases compare every output; full-size workloads
compare whole sampled heads (the oracle is run on that head alone)."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from fibonacci_offset_transformer_amd import fsa, schedules, synth

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2}


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def inputs(workload, layer, shape, dtype, grad=False):
    t = synth.layer_inputs(workload, layer, shape, dtype, with_grad=grad)
    return {k: v.to(dev()) for k, v in t.items()}


def maxabs(gpu, ref):
    return float(np.max(np.abs(synth.as_f64(gpu) - ref))) if ref.size else 0.0


def check(name, gpu, ref, tol):
    err = maxabs(gpu, ref)
    note(f"  {name}: max|err|={err:.3e} max|ref|={float(np.max(np.abs(ref))) if ref.size else 0:.3f} tol={tol}")
    assert err <= tol, (name, err)


def same_rounding(name, lo, f32):
    """A low-precision output must be the round-to-nearest-even image of the float32 output."""
    assert torch.equal(lo, f32.to(lo.dtype)), name


def fwd_case(workload, B, H, N, dtype, base, alpha, w, R, heads=None, layer=0):
    """Runs the forward with float32 outputs (checked against the oracle at the dtype's bar) and
    with outputs in the input dtype (checked to be the rounding of the float32 outputs)."""
    scale = 1.0 / math.sqrt(64)
    x = inputs(workload, layer, (B, H, N, 64), dtype)
    note(f"forward wl={workload} layer={layer} {dtype} B={B} H={H} N={N} base={base} alpha={alpha} w={w} R={R}")
    kw = dict(alpha=alpha, w=w, R=R, base=base, scale=scale)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], out_dtype=torch.float32, **kw)
    o_lo, lse_lo = fsa.forward(x["q"], x["k"], x["v"], out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    same_rounding("o", o_lo, o)
    assert torch.equal(lse_lo, lse)
    T = oracle.offset_table(base, alpha, w, R)
    assert fsa.build_offsets(alpha, w, R, base) == T
    sel = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in sel:
        q, k, v = (synth.as_f64(x[t][b, h]) for t in ("q", "k", "v"))
        ro, rl = oracle.sparse_forward(q, k, v, T, w, scale)
        check(f"o[{b},{h}]", o[b, h], ro, TOL[dtype])
        check(f"lse[{b},{h}]", lse[b, h], rl, TOL[dtype])
    return x, o_lo if dtype == torch.bfloat16 else o, lse


def bwd_case(workload, B, H, N, dtype, base, alpha, w, R, heads=None, layer=0):
    """Forward in the input dtype (its O feeds the backward), then the backward with float32
    gradients (checked against the oracle) and with input-dtype gradients (checked to be the
    rounding of the float32 ones)."""
    scale = 1.0 / math.sqrt(64)
    x = inputs(workload, layer, (B, H, N, 64), dtype, grad=True)
    note(f"backward wl={workload} layer={layer} {dtype} B={B} H={H} N={N} base={base} alpha={alpha} w={w} R={R}")
    kw = dict(alpha=alpha, w=w, R=R, base=base, scale=scale)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], **kw)
    g = fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], out_dtype=torch.float32, **kw)
    g_lo = fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), g_lo, g):
        same_rounding(name, a, b)
    T = oracle.offset_table(base, alpha, w, R)
    sel = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in sel:
        q, k, v, do = (synth.as_f64(x[t][b, h]) for t in ("q", "k", "v", "do"))
        rq, rk, rv = oracle.sparse_backward(q, k, v, do, T, w, scale)
        check(f"dq[{b},{h}]", g[0][b, h], rq, TOL[dtype])
        check(f"dk[{b},{h}]", g[1][b, h], rk, TOL[dtype])
        check(f"dv[{b},{h}]", g[2][b, h], rv, TOL[dtype])
    return x, (o, lse), g


# ---------------------------------------------------------------- small, exhaustive

SMALL = [
    # (N, base, alpha, w, R)
    (1, "fib", 1.0, 16, 256),
    (17, "fib", 1.0, 16, 256),
    (100, "fib", 1.0, 6, 256),
    (300, "fib", 1.0, 16, 256),
    (300, "fib", 0.5, 8, 256),
    (300, "fib", 1.5, 12, 256),
    (300, "fib", 1.0, 64, 1024),
    (300, "pow2", 1.0, 10, 1024),
    (300, "fib", 1.0, 100, 256),     # window wider than a tile
    (257, "fib", 1.0, 1, 1024),      # no window besides self, every Fibonacci offset
    (130, "fib", 1.0, 300, 1024),    # window covers the whole sequence (dense)
    (1100, "fib", 1.0, 6, 1024),     # 11 offsets: more than the unrolled slots, 16 pair slots
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("N,base,alpha,w,R", SMALL)
def test_forward_small(dtype, N, base, alpha, w, R):
    fwd_case(11, 1, 2, N, dtype, base, alpha, w, R)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("N,base,alpha,w,R", SMALL)
def test_backward_small(dtype, N, base, alpha, w, R):
    bwd_case(12, 1, 2, N, dtype, base, alpha, w, R)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_window_one_empty_table_returns_v(dtype):
    x = inputs(13, 0, (2, 3, 150, 64), dtype)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], alpha=1.0, w=1, R=1, scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(o, x["v"])
    ref = 0.125 * (x["q"].double() * x["k"].double()).sum(-1)
    assert float((lse.double() - ref).abs().max()) <= 1e-5


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_wide_window_equals_dense_kernel_and_oracle(dtype):
    x = inputs(14, 0, (1, 2, 200, 64), dtype)
    o, l = fsa.forward(x["q"], x["k"], x["v"], alpha=1.0, w=200, R=1024, scale=0.125, out_dtype=torch.float32)
    od, ld = fsa.dense_forward(x["q"], x["k"], x["v"], scale=0.125, out_dtype=torch.float32)
    od_lo, _ = fsa.dense_forward(x["q"], x["k"], x["v"], scale=0.125)
    torch.cuda.synchronize()
    same_rounding("dense o", od_lo, od)
    for h in range(2):
        q, k, v = (synth.as_f64(x[t][0, h]) for t in ("q", "k", "v"))
        ro, rl = oracle.dense_forward(q, k, v, 0.125)
        check(f"dense o[{h}]", od[0, h], ro, TOL[dtype])
        check(f"dense lse[{h}]", ld[0, h], rl, TOL[dtype])
        check(f"wide o[{h}]", o[0, h], ro, TOL[dtype])


@pytest.mark.parametrize("N,scale", [(1, 0.125), (17, 0.125), (64, 0.125), (65, 0.125), (128, 0.125),
                                     (129, 0.125), (191, 0.125), (256, 0.125), (333, 0.125), (1000, 0.125),
                                     (333, -0.125), (200, 0.0)])
def test_dense_forward_against_oracle(N, scale):
    # bf16 with a positive scale takes the dedicated dense kernel; other scales the general one
    x = inputs(15, 0, (1, 3, N, 64), torch.bfloat16)
    od, ld = fsa.dense_forward(x["q"], x["k"], x["v"], scale=scale, out_dtype=torch.float32)
    od_lo, ld_lo = fsa.dense_forward(x["q"], x["k"], x["v"], scale=scale)
    torch.cuda.synchronize()
    same_rounding("dense o", od_lo, od)
    assert torch.equal(ld_lo, ld)
    for h in range(3):
        q, k, v = (synth.as_f64(x[t][0, h]) for t in ("q", "k", "v"))
        ro, rl = oracle.dense_forward(q, k, v, scale)
        check(f"dense o[0,{h}] N={N} scale={scale}", od[0, h], ro, TOL[torch.bfloat16])
        check(f"dense lse[0,{h}] N={N} scale={scale}", ld[0, h], rl, TOL[torch.bfloat16])


def test_empty_problem_is_noop():
    q = torch.empty((2, 3, 0, 64), dtype=torch.bfloat16, device=dev())
    o, l = fsa.forward(q, q.clone(), q.clone(), alpha=1.0, w=64, R=1024)
    assert o.shape == q.shape and l.shape == (2, 3, 0)


def test_unsupported_head_size_raises():
    q = torch.zeros((1, 1, 16, 32), dtype=torch.bfloat16, device=dev())
    with pytest.raises(fsa.FsaError) as e:
        fsa.forward(q, q.clone(), q.clone(), alpha=1.0, w=64, R=1024)
    assert e.value.status == fsa.FSA_E_UNSUPPORTED


# ---------------------------------------------------------------- full-size workloads

def test_workload1_single_head_fp32():
    # fp32 [1,1,256,64], w=16, alpha=1, R=256, forward
    fwd_case(1, 1, 1, 256, torch.float32, "fib", 1.0, 16, 256)


def test_workload2_one_layer_bf16():
    # bf16 [8,8,1024,64], w=64, alpha=1, R=1024, forward; every head compared
    fwd_case(2, 8, 8, 1024, torch.bfloat16, "fib", 1.0, 64, 1024)


def test_workload3_sixteen_layer_stagger_forward():
    alphas = schedules.linear_stagger(16)
    rng = np.random.default_rng(3)
    for l, a in enumerate(alphas):
        b, h = (int(z) for z in rng.integers(0, 8, 2))
        fwd_case(3, 8, 8, 1024, torch.bfloat16, "fib", a, 64, 1024, heads=[(b, h)], layer=l)


def test_workload4_training_step_at_4096():
    alphas = schedules.linear_stagger(16)
    rng = np.random.default_rng(4)
    for l in range(16):
        b, h = int(rng.integers(0, 2)), int(rng.integers(0, 8))
        fwd_case(4, 2, 8, 4096, torch.bfloat16, "fib", alphas[l], 64, 1024, heads=[(b, h)], layer=l)
        bwd_case(4, 2, 8, 4096, torch.bfloat16, "fib", alphas[l], 64, 1024, heads=[(b, h)], layer=l)


def test_workload4_dense_baseline_sampled_rows():
    x = inputs(4, 0, (2, 8, 4096, 64), torch.bfloat16)
    od, ld = fsa.dense_forward(x["q"], x["k"], x["v"], scale=0.125, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, 1000, 2047, 4000, 4095])
    for b, h in ((0, 0), (1, 7)):
        q, k, v = (synth.as_f64(x[t][b, h]) for t in ("q", "k", "v"))
        ro, rl = oracle.dense_forward_rows(q, k, v, 0.125, rows)
        check(f"dense o[{b},{h}] rows", od[b, h][rows], ro, 1e-2)
        check(f"dense lse[{b},{h}] rows", ld[b, h][rows], rl, 1e-2)


def test_workload5_long_context_pow2():
    fwd_case(5, 1, 8, 32768, torch.bfloat16, "pow2", 1.0, 64, 1024, heads=[(0, 3)])
    bwd_case(5, 1, 8, 32768, torch.bfloat16, "pow2", 1.0, 64, 1024, heads=[(0, 3)])


# ---------------------------------------------------------------- properties

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_bitwise_deterministic(dtype):
    x = inputs(15, 0, (2, 4, 1000, 64), dtype, grad=True)
    kw = dict(alpha=1.5, w=64, R=1024, scale=0.125)
    a = fsa.forward(x["q"], x["k"], x["v"], **kw)
    b = fsa.forward(x["q"], x["k"], x["v"], **kw)
    ga = fsa.backward(x["q"], x["k"], x["v"], a[0], a[1], x["do"], **kw)
    gb = fsa.backward(x["q"], x["k"], x["v"], a[0], a[1], x["do"], **kw)
    torch.cuda.synchronize()
    for u, v in zip(a + ga, b + gb):
        assert torch.equal(u, v)


def test_prefix_rows_unchanged_when_sequence_grows():
    # rows < 1024 of an N=4096 run equal an N=1024 run on the prefix (1024 -> 4096 protocol)
    x = inputs(16, 0, (1, 4, 4096, 64), torch.bfloat16)
    kw = dict(alpha=1.0, w=64, R=1024, scale=0.125)
    o, l = fsa.forward(x["q"], x["k"], x["v"], **kw)
    p = {t: x[t][:, :, :1024].contiguous() for t in ("q", "k", "v")}
    op, lp = fsa.forward(p["q"], p["k"], p["v"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, :1024], op)
    assert torch.equal(l[:, :, :1024], lp)


def test_outputs_leave_guard_bands_untouched():
    x = inputs(17, 0, (1, 2, 333, 64), torch.bfloat16, grad=True)
    n = x["q"].numel()
    canary = 12345.0
    big = torch.full((n + 2048,), canary, dtype=torch.bfloat16, device=dev())
    o = big[1024:1024 + n].view(x["q"].shape)
    lbig = torch.full((666 + 2048,), canary, dtype=torch.float32, device=dev())
    lse = lbig[1024:1024 + 666].view(1, 2, 333)
    fsa.forward(x["q"], x["k"], x["v"], alpha=1.0, w=64, R=1024, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool((big[:1024] == canary).all()) and bool((big[1024 + n:] == canary).all())
    assert bool((lbig[:1024] == canary).all()) and bool((lbig[1024 + 666:] == canary).all())


def test_backward_equals_its_two_stages():
    x = inputs(18, 0, (1, 3, 500, 64), torch.bfloat16, grad=True)
    kw = dict(alpha=0.9, w=64, R=1024, scale=0.125)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], **kw)
    whole = fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], **kw)
    D = fsa.backward_delta(o, x["do"])
    parts = fsa.backward_grads(x["q"], x["k"], x["v"], lse, x["do"], D, **kw)
    torch.cuda.synchronize()
    for a, b in zip(whole, parts):
        assert torch.equal(a, b)
    ref = (o.double() * x["do"].double()).sum(-1)
    assert float((D.double() - ref).abs().max()) <= 1e-4


@pytest.mark.parametrize("scale", [-0.125, 0.0, 1e-3])
def test_forward_any_scale(scale):
    # the window kernel takes positive scales; others run the general kernel
    x = inputs(21, 0, (1, 2, 300, 64), torch.bfloat16)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], alpha=1.0, w=64, R=1024, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    T = oracle.offset_table("fib", 1.0, 64, 1024)
    for h in range(2):
        q, k, v = (synth.as_f64(x[t][0, h]) for t in ("q", "k", "v"))
        ro, rl = oracle.sparse_forward(q, k, v, T, 64, scale)
        check(f"o[0,{h}] scale={scale}", o[0, h], ro, TOL[torch.bfloat16])
        check(f"lse[0,{h}] scale={scale}", lse[0, h], rl, TOL[torch.bfloat16])


@pytest.mark.parametrize("H", [2, 8], ids=["two_kernels", "one_launch"])
def test_pair_workspace_contents_do_not_matter(H):
    # every word the dK/dV work reads was written by the dQ work of the same call
    x = inputs(20, 0, (1, H, 777, 64), torch.bfloat16, grad=True)
    kw = dict(alpha=0.75, w=64, R=1024, scale=0.125)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], **kw)
    need = fsa.workspace_bytes(torch.bfloat16, 1, H, 777, alpha=0.75, w=64, R=1024)
    assert need > 0
    runs = []
    for fill in (0, 0x7FC07FC0, -1):  # zeros, NaN bit patterns, all ones
        pw = torch.full((need // 4 + 333,), fill, dtype=torch.int32, device=dev())
        runs.append(fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], pair_ws=pw, out_dtype=torch.float32, **kw))
    torch.cuda.synchronize()
    for other in runs[1:]:
        for a, b in zip(runs[0], other):
            assert torch.equal(a, b)
    T = oracle.offset_table("fib", 0.75, 64, 1024)
    for h in range(H):
        q, k, v, do = (synth.as_f64(x[t][0, h]) for t in ("q", "k", "v", "do"))
        for name, got, want in zip(("dq", "dk", "dv"), runs[0], oracle.sparse_backward(q, k, v, do, T, 64, 0.125)):
            check(f"{name}[0,{h}]", got[0, h], want, TOL[torch.bfloat16])


@pytest.mark.parametrize("N,alpha,w", [(65, 1.0, 64), (777, 0.75, 64), (1500, 1.4, 64),
                                       (1100, 1.0, 1)])  # the last: 15 offsets, 16 pair slots
def test_one_launch_backward_equals_per_head_backward(N, alpha, w):
    # B * H a multiple of 8 takes the one-launch backward (dK/dV tiles wait for the dQ
    # tiles' tokens); one head at a time takes the two-kernel path: the same arithmetic
    # per tile, so the results agree bit for bit
    x = inputs(22, 0, (2, 4, N, 64), torch.bfloat16, grad=True)
    kw = dict(alpha=alpha, w=w, R=1024, scale=0.125)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], **kw)
    note(f"one-launch backward N={N} alpha={alpha} w={w}")
    whole = fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], out_dtype=torch.float32, **kw)
    D = fsa.backward_delta(o, x["do"])
    staged = fsa.backward_grads(x["q"], x["k"], x["v"], lse, x["do"], D, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(4):
            one = {t: x[t][b:b + 1, h:h + 1].clone() for t in ("q", "k", "v", "do")}
            ref = fsa.backward(one["q"], one["k"], one["v"], o[b:b + 1, h:h + 1].clone(),
                               lse[b:b + 1, h:h + 1].clone(), one["do"], out_dtype=torch.float32, **kw)
            torch.cuda.synchronize()
            for name, a, a2, r in zip(("dq", "dk", "dv"), whole, staged, ref):
                assert torch.equal(a[b, h], r[0, 0]), (name, b, h)
                assert torch.equal(a2[b, h], r[0, 0]), (name, b, h, "staged")
    # and one head against the oracle
    T = oracle.offset_table("fib", alpha, w, 1024)
    q, k, v, do = (synth.as_f64(x[t][1, 3]) for t in ("q", "k", "v", "do"))
    for name, got, want in zip(("dq", "dk", "dv"), whole, oracle.sparse_backward(q, k, v, do, T, w, 0.125)):
        check(f"{name}[1,3]", got[1, 3], want, TOL[torch.bfloat16])


def test_one_launch_backward_reused_workspace():
    # consecutive calls on one workspace with different inputs, on two streams: each call
    # waits for its own launch's tokens, never an earlier call's (whose pair words differ)
    kw = dict(alpha=1.1, w=64, R=1024, scale=0.125)
    need = fsa.workspace_bytes(torch.bfloat16, 1, 8, 900, alpha=1.1, w=64, R=1024)
    pw = torch.full((need // 4,), -1, dtype=torch.int32, device=dev())
    other = torch.cuda.Stream()
    for seed in (23, 24, 25, 26):
        x = inputs(seed, 0, (1, 8, 900, 64), torch.bfloat16, grad=True)
        o, lse = fsa.forward(x["q"], x["k"], x["v"], **kw)
        fresh = fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], **kw)
        torch.cuda.synchronize()
        s = other if seed % 2 else torch.cuda.current_stream()
        with torch.cuda.stream(s):
            got = fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], pair_ws=pw, **kw)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, fresh):
            assert torch.equal(a, b), (seed, name)
            assert bool(torch.isfinite(a.float()).all()), (seed, name)


def test_graph_replays_match_eager():
    x = inputs(19, 0, (2, 4, 700, 64), torch.bfloat16, grad=True)
    kw = dict(alpha=1.2, w=64, R=1024, scale=0.125)
    bufs = {n: torch.empty_like(x["q"]) for n in ("o", "dq", "dk", "dv")}
    lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device=x["q"].device)
    D = torch.empty_like(lse)
    pw = torch.empty(fsa.workspace_bytes(torch.bfloat16, 2, 4, 700, w=64, R=1024, alpha=1.2) // 4,
                     dtype=torch.int32, device=x["q"].device)

    def step():
        fsa.forward(x["q"], x["k"], x["v"], out=bufs["o"], lse=lse, **kw)
        fsa.backward(x["q"], x["k"], x["v"], bufs["o"], lse, x["do"], dq=bufs["dq"], dk=bufs["dk"],
                     dv=bufs["dv"], delta=D, pair_ws=pw, **kw)

    step()
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in bufs.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in bufs.values():
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in bufs:
            assert torch.equal(bufs[n], ref[n]), (rep, n)


# ---------------------------------------------------------------- decode (one query per sequence)

def decode_case(dtype, base, alpha, w, R, lens, Lmax=700, H=2, scale=0.125, seed=30):
    """fsa.decode on a ragged batch against the oracle's forward row L - 1 of each cache."""
    B = len(lens)
    x = inputs(seed, 0, (B, H, Lmax, 64), dtype, grad=True)  # k, v are the caches; dO rows serve as queries
    q = x["do"][:, :, 0, :].contiguous()
    sl = torch.tensor(lens, dtype=torch.int32, device=dev())
    note(f"decode {dtype} base={base} alpha={alpha} w={w} R={R} lens={lens} Lmax={Lmax}")
    o, lse = fsa.decode(q, x["k"], x["v"], sl, alpha=alpha, w=w, R=R, base=base, scale=scale,
                        out_dtype=torch.float32)
    o_lo, lse_lo = fsa.decode(q, x["k"], x["v"], sl, alpha=alpha, w=w, R=R, base=base, scale=scale)
    torch.cuda.synchronize()
    same_rounding("decode o", o_lo, o)
    assert torch.equal(lse_lo, lse)
    T = oracle.offset_table(base, alpha, w, R)
    for b, L in enumerate(lens):
        L = min(max(L, 1), Lmax)
        for h in range(H):
            k, v = (synth.as_f64(x[t][b, h, :L]) for t in ("k", "v"))
            qf = np.zeros_like(k)
            qf[L - 1] = synth.as_f64(q[b, h])
            ro, rl = oracle.sparse_forward_rows(qf, k, v, T, w, scale, [L - 1])
            check(f"decode o[{b},{h}] L={L}", o[b, h][None], ro, TOL[dtype])
            check(f"decode lse[{b},{h}] L={L}", lse[b, h][None], rl, TOL[dtype])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("base,alpha,w,R", [("fib", 1.0, 64, 1024), ("fib", 1.5, 16, 1024), ("pow2", 1.0, 64, 1024),
                                             ("fib", 0.5, 1, 256)])
def test_decode_against_oracle(dtype, base, alpha, w, R):
    decode_case(dtype, base, alpha, w, R, [1, 5, 64, 65, 333, 700])


def test_decode_dense_window_and_clamped_lengths():
    # a window covering the cache is dense decoding; lengths outside [1, Lmax] are clamped
    decode_case(torch.bfloat16, "fib", 1.0, 700, 1024, [700, 1, 250])
    decode_case(torch.bfloat16, "fib", 1.0, 64, 1024, [0, -3, 9999, 700])


def test_decode_matches_forward_last_row():
    x = inputs(31, 0, (2, 4, 1000, 64), torch.bfloat16)
    kw = dict(alpha=1.2, w=64, R=1024, scale=0.125)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], out_dtype=torch.float32, **kw)
    sl = torch.full((2,), 1000, dtype=torch.int32, device=dev())
    od, ld = fsa.decode(x["q"][:, :, -1].contiguous(), x["k"], x["v"], sl, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    assert float((od - o[:, :, -1]).abs().max()) <= 1e-2
    assert float((ld - lse[:, :, -1]).abs().max()) <= 1e-2


# ---------------------------------------------------------------- the pages' other schedules

@pytest.mark.parametrize("layer", [0, 5, 11, 15])
def test_coprime_stagger_layers(layer):
    # the coprime reassignment gives layer l the linear-stagger alpha of layer 7 l mod 16
    alpha = schedules.coprime_stagger(16)[layer]
    assert alpha == schedules.linear_stagger(16)[oracle.coprime_layer(layer)]
    bwd_case(32, 1, 2, 1500, torch.bfloat16, "fib", alpha, 64, 1024, layer=layer)


@pytest.mark.parametrize("layer", [0, 8, 15])
def test_pow2_base_with_stagger(layer):
    alpha = schedules.linear_stagger(16)[layer]
    bwd_case(33, 1, 2, 1200, torch.bfloat16, "pow2", alpha, 64, 1024, layer=layer)


@pytest.mark.parametrize("w", [6, 8, 10, 12])
def test_window_sweep(w):
    # the pages' window sweep with the Fibonacci table (offsets below w join the window)
    fwd_case(34, 1, 2, 700, torch.bfloat16, "fib", 1.0, w, 1024)
    bwd_case(34, 1, 2, 700, torch.bfloat16, "fib", 1.0, w, 1024)


@pytest.mark.parametrize("layer", [3, 14, 15])
def test_literal_stagger_formula_layers(layer):
    # alpha_l = 0.5 + l*(1.5/15) as one workload description writes it: up to 8 offsets
    # (the largest 1974) at the training-step shape
    a = schedules.literal_stagger(16)[layer]
    T = oracle.offset_table("fib", a, 64, 1024)
    assert fsa.build_offsets(a, 64, 1024) == T
    rng = np.random.default_rng(70 + layer)
    b, h = int(rng.integers(0, 2)), int(rng.integers(0, 8))
    fwd_case(7, 2, 8, 4096, torch.bfloat16, "fib", a, 64, 1024, heads=[(b, h)], layer=layer)
    bwd_case(7, 2, 8, 4096, torch.bfloat16, "fib", a, 64, 1024, heads=[(b, h)], layer=layer)


def test_pow2_reach_at_evaluation_length():
    # the power-of-2 control with its reach at the evaluation length (R = N = 4096): the
    # table gains 1024 and 2048, the large offsets that control brought in at 4x length
    T = oracle.offset_table("pow2", 1.0, 64, 4096)
    assert T == [64, 128, 256, 512, 1024, 2048] and fsa.build_offsets(1.0, 64, 4096, "pow2") == T
    fwd_case(35, 2, 8, 4096, torch.bfloat16, "pow2", 1.0, 64, 4096, heads=[(0, 2), (1, 7)])
    bwd_case(35, 2, 8, 4096, torch.bfloat16, "pow2", 1.0, 64, 4096, heads=[(1, 5)])


def test_fibonacci_reach_at_evaluation_length():
    # the Fibonacci table with its reach at the evaluation length (R = N = 4096) at the
    # stagger's largest alpha: base values up to 2584 give offsets up to 3876, nine
    # entries (one past the kernels' unrolled slab groups)
    T = oracle.offset_table("fib", 1.5, 64, 4096)
    assert len(T) == 9 and T[-1] == 3876 and fsa.build_offsets(1.5, 64, 4096, "fib") == T
    fwd_case(36, 2, 8, 4096, torch.bfloat16, "fib", 1.5, 64, 4096, heads=[(0, 3), (1, 6)])
    bwd_case(36, 2, 8, 4096, torch.bfloat16, "fib", 1.5, 64, 4096, heads=[(0, 1)])


@pytest.mark.parametrize("layer", [0, 9, 15])
def test_workload4_edge_tiles_of_every_head(layer):
    # the first and last 64-row tiles of all 16 heads of a training-step layer (the
    # sequence start and end, where masks and buffer ranges cut the tiles), row by row
    alpha = schedules.linear_stagger(16)[layer]
    x = inputs(4, layer, (2, 8, 4096, 64), torch.bfloat16, grad=True)
    kw = dict(alpha=alpha, w=64, R=1024, scale=0.125)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], **kw)
    o32, _ = fsa.forward(x["q"], x["k"], x["v"], out_dtype=torch.float32, **kw)
    g = fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    T = oracle.offset_table("fib", alpha, 64, 1024)
    rows = np.concatenate([np.arange(0, 64), np.arange(4096 - 64, 4096)])
    note(f"edge tiles of every head, layer {layer} alpha={alpha:.4f}")
    worst = 0.0
    for b in range(2):
        for h in range(8):
            q, k, v, do = (synth.as_f64(x[t][b, h]) for t in ("q", "k", "v", "do"))
            ro, rl = oracle.sparse_forward_rows(q, k, v, T, 64, 0.125, rows)
            rq, rk, rv = oracle.sparse_backward_rows(q, k, v, do, T, 64, 0.125, rows)
            for name, got, want in (("o", o32[b, h][rows], ro), ("lse", lse[b, h][rows], rl),
                                    ("dq", g[0][b, h][rows], rq), ("dk", g[1][b, h][rows], rk),
                                    ("dv", g[2][b, h][rows], rv)):
                err = maxabs(got, want)
                worst = max(worst, err)
                assert err <= 1e-2, (b, h, name, err)
    note(f"  worst max|err| over all heads' edge tiles: {worst:.3e}")


def test_binding_rejects_bad_row_buffers():
    # LSE and D are float32 [B, H, N] on the inputs' device, contiguous; anything else is
    # refused before any kernel runs
    x = inputs(36, 0, (1, 2, 100, 64), torch.bfloat16, grad=True)
    kw = dict(alpha=1.0, w=64, R=1024)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], **kw)
    bad = [lse[:, :1], lse.to(torch.bfloat16), lse.cpu(), torch.empty(1, 100, 2, device=dev()).transpose(1, 2),
           torch.empty(2, 100, device=dev())]
    for b in bad:
        with pytest.raises(ValueError):
            fsa.forward(x["q"], x["k"], x["v"], lse=b, **kw)
        with pytest.raises(ValueError):
            fsa.backward(x["q"], x["k"], x["v"], o, b, x["do"], **kw)
        with pytest.raises(ValueError):
            fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], delta=b, **kw)
        with pytest.raises(ValueError):
            fsa.backward_grads(x["q"], x["k"], x["v"], b, x["do"], lse, **kw)
        with pytest.raises(ValueError):
            fsa.frac_backward(x["q"], x["k"], x["v"], o, b, x["do"], **kw)
    with pytest.raises(ValueError):
        fsa.backward(x["q"], x["k"], x["v"], o, None, x["do"], **kw)
    # decode: LSE is [B, H]
    q1 = x["q"][:, :, -1].contiguous()
    sl = torch.full((1,), 100, dtype=torch.int32, device=dev())
    with pytest.raises(ValueError):
        fsa.decode(q1, x["k"], x["v"], sl, lse=torch.empty((1, 2, 1), device=dev()), **kw)
    with pytest.raises(ValueError):
        fsa.decode(q1, x["k"], x["v"], sl, out=torch.empty((1, 2, 32), device=dev(), dtype=torch.bfloat16), **kw)


# ---------------------------------------------------------------- sharp attention, small windows

@pytest.mark.parametrize("H", [3, 8], ids=["two_kernels", "one_launch"])
def test_small_window_backward_with_sharp_attention(H):
    # scale 1/2 (attention logits of standard deviation about 4) at w = 8: single keys take
    # most of a row's weight, where one bf16 rounding of a pair's P and dS would move a
    # gradient by up to about 0.02; the fp32 pair slots below w = 64 keep it within 1e-2.
    # The backward is handed the oracle's own O (bf16) and LSE, as in the sweep
    B, N, w, alpha, R, scale = 1, 400, 8, 1.0, 1024, 0.5
    x = inputs(41, 0, (B, H, N, 64), torch.bfloat16, grad=True)
    T = oracle.offset_table("fib", alpha, w, R)
    o_ref, lse_ref = np.zeros((B, H, N, 64)), np.zeros((B, H, N))
    for h in range(H):
        q, k, v = (synth.as_f64(x[t][0, h]) for t in ("q", "k", "v"))
        o_ref[0, h], lse_ref[0, h] = oracle.sparse_forward(q, k, v, T, w, scale)
    o_in = torch.from_numpy(o_ref).to(torch.bfloat16)
    lse_in = torch.from_numpy(lse_ref).to(torch.float32)
    g = fsa.backward(x["q"], x["k"], x["v"], o_in.to(dev()), lse_in.to(dev()), x["do"], alpha=alpha, w=w, R=R,
                     scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    note(f"sharp attention backward B={B} H={H} N={N} w={w} scale={scale}")
    og, lg = synth.as_f64(o_in), synth.as_f64(lse_in)
    for h in range(H):
        q, k, v, do = (synth.as_f64(x[t][0, h]) for t in ("q", "k", "v", "do"))
        ref = oracle.sparse_backward(q, k, v, do, T, w, scale, o=og[0, h], lse=lg[0, h])
        for name, got, want in zip(("dq", "dk", "dv"), g, ref):
            check(f"{name}[{h}]", got[0, h], want, 1e-2)
