"""The window kernels at the largest sizes they take, row by row against the oracle.

N = 2^24 is the longest sequence the bf16 window kernels accept: a head's rows then
span exactly 2^31 bytes, the limit of the per-head buffer descriptors. A second case
runs the one-launch backward (B * H = 8) over 262 144 tiles, far more than the GPU
holds at once, so its dK/dV tiles are dispatched long after the first dQ tiles ended.

Inputs are N(0, 1) draws from a seeded generator on the device. The oracle sees, for
each sampled row, the slice of rows that can influence it: for a query row i, keys
i - M .. i (M the largest attended offset); for dK and dV of key row j, the queries
j .. j + M and their keys, so rows j - M .. j + M. Row indices inside the slice are
shifted, which changes nothing since every attended key lies inside it."""
import sys

import numpy as np
import pytest
import torch

import oracle
from fibonacci_offset_transformer_amd import fsa, synth

pytestmark = pytest.mark.gpu


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def slice_rows(x, lo, hi):
    return synth.as_f64(x[lo:hi])


def run_case(seed, B, H, N, rows, alpha=1.0, w=64, R=1024, scale=0.125):
    shape = (B, H, N, 64)
    note(f"large case B={B} H={H} N={N} alpha={alpha} w={w} R={R}: drawing inputs")
    x = {t: synth.normal_on(dev(), shape, synth.seed_of(90 + seed, 0, t), torch.bfloat16) for t in ("q", "k", "v", "do")}
    kw = dict(alpha=alpha, w=w, R=R, scale=scale)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], **kw)
    o32, _ = fsa.forward(x["q"], x["k"], x["v"], out_dtype=torch.float32, **kw)
    g = fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    note("  kernels done; checking sampled rows")
    T = oracle.offset_table("fib", alpha, w, R)
    M = max([w - 1] + [o_ for o_ in T if o_ < N])
    worst = 0.0
    for b in range(B):
        for h in range(H):
            for j in rows:
                lo, hi = max(0, j - M), min(N, j + M + 1)
                q, k, v, do = (slice_rows(x[t][b, h], lo, hi) for t in ("q", "k", "v", "do"))
                r = j - lo
                ro, rl = oracle.sparse_forward_rows(q, k, v, T, w, scale, [r])
                rq, rk, rv = oracle.sparse_backward_rows(q, k, v, do, T, w, scale, [r])
                for name, got, want in (("o", o32[b, h, j], ro[0]), ("lse", lse[b, h, j], rl[0]),
                                        ("dq", g[0][b, h, j], rq[0]), ("dk", g[1][b, h, j], rk[0]),
                                        ("dv", g[2][b, h, j], rv[0])):
                    err = float(np.max(np.abs(synth.as_f64(got) - want)))
                    worst = max(worst, err)
                    assert err <= 1e-2, (b, h, j, name, err)
    note(f"  worst max|err| over {B * H * len(rows)} sampled rows: {worst:.3e}")


def test_longest_sequence_of_the_window_kernels():
    N = 1 << 24
    rows = [0, 1, 63, 64, 1000, (1 << 23) - 1, 1 << 23, (1 << 23) + 777, N - 1000, N - 65, N - 64, N - 2, N - 1]
    run_case(1, 1, 1, N, rows)


def test_one_launch_backward_over_many_tiles():
    N = 1 << 21
    rows = [0, 65, 5000, 1 << 20, N - 999, N - 1]
    run_case(2, 1, 8, N, rows, alpha=1.3)
