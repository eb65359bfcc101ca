"""fsa_backward_noalloc through the C ABI: the backward with its workspaces (D, pair
weights, tokens, status word) in the library's static device scratch, for callers that
cannot allocate. It runs the same kernels as fsa_backward, so its gradients must equal
fsa_backward's bit for bit: checked on two calls in a row, the second smaller (the
scratch keeps the first call's contents), on the one-launch, two-kernel, fp32-slot
(narrow window) and general (fp32 inputs) paths, under HIP graph capture, and with a
problem too large for the scratch, which is refused before anything runs."""
import ctypes
import sys

import pytest
import torch

from fibonacci_offset_transformer_amd import fsa, synth

pytestmark = pytest.mark.gpu


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def noalloc(q, k, v, o, lse, do, dq, dk, dv, alpha, w, R, base="fib", scale=0.125):
    """The C entry point, called directly (ctypes), into preallocated outputs."""
    B, H, N, d = q.shape
    L = fsa.library()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    return L.fsa_backward_noalloc(fsa.DTYPES[q.dtype], fsa.DTYPES[dq.dtype], p(q), p(k), p(v), p(o), p(lse), p(do),
                                  p(dq), p(dk), p(dv), B, H, N, d, scale, fsa.BASES[base], float(alpha), int(w),
                                  int(R), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def case(seed, shape, dtype, alpha, w, R, base="fib"):
    x = {k: t.to(dev()) for k, t in synth.layer_inputs(seed, 0, shape, dtype, with_grad=True).items()}
    kw = dict(alpha=alpha, w=w, R=R, base=base, scale=0.125)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], **kw)
    want = fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], out_dtype=torch.float32, **kw)
    got = [torch.full(x["q"].shape, float("nan"), dtype=torch.float32, device=dev()) for _ in range(3)]
    st = noalloc(x["q"], x["k"], x["v"], o, lse, x["do"], *got, alpha, w, R, base)
    assert st == fsa.FSA_OK, fsa.library().fsa_last_error()
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        assert torch.equal(a, b), name
    assert not fsa.wait_status("backward_noalloc", x["q"], None, alpha=alpha, w=w, R=R, base=base)
    return x


@pytest.mark.parametrize("first,second", [
    # one-launch backward, then a smaller one-launch problem
    (((2, 8, 4096, 64), torch.bfloat16, 1.5, 64, 1024), ((1, 8, 700, 64), torch.bfloat16, 0.8, 64, 1024)),
    # one-launch, then a smaller two-kernel problem with fp32 pair slots (narrow window)
    (((1, 8, 2000, 64), torch.bfloat16, 1.0, 64, 1024), ((1, 3, 500, 64), torch.bfloat16, 1.2, 5, 1024)),
    # fp32 pair slots in one launch, then the general kernels (fp32 inputs: D only)
    (((2, 4, 1500, 64), torch.bfloat16, 0.9, 8, 1024), ((1, 2, 300, 64), torch.float32, 1.0, 16, 256)),
])
def test_noalloc_equals_backward_on_two_calls(first, second):
    for i, (shape, dtype, alpha, w, R) in enumerate((first, second)):
        note(f"call {i}: {shape} {dtype} alpha={alpha} w={w} R={R}")
        case(200 + i, shape, dtype, alpha, w, R)


def test_noalloc_in_a_graph_matches_eager():
    x = {k: t.to(dev()) for k, t in synth.layer_inputs(210, 0, (1, 8, 900, 64), torch.bfloat16,
                                                       with_grad=True).items()}
    kw = dict(alpha=1.1, w=64, R=1024, scale=0.125)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], **kw)
    want = fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], **kw)
    out = [torch.empty_like(x["q"]) for _ in range(3)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        assert noalloc(x["q"], x["k"], x["v"], o, lse, x["do"], *out, 1.1, 64, 1024) == fsa.FSA_OK
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert noalloc(x["q"], x["k"], x["v"], o, lse, x["do"], *out, 1.1, 64, 1024) == fsa.FSA_OK
    for rep in range(3):
        for t in out:
            t.zero_()
        # another call between replays leaves other contents in the scratch
        case(211 + rep, (1, 8, 300, 64), torch.bfloat16, 1.3, 64, 1024)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), out, want):
            assert torch.equal(a, b), (rep, name)


def test_noalloc_refuses_problems_beyond_the_scratch():
    # [1,8,32768,64] at w = 64: D 1 MiB plus 8 pair slots per row (8 MiB) fits; at w = 8
    # with R = 2^16 the slots carry fp32 pairs and 18 offsets lie below N (24 slots): the
    # 48 MiB of pair words alone do not fit
    x = {k: t.to(dev()) for k, t in synth.layer_inputs(220, 0, (1, 8, 32768, 64), torch.bfloat16,
                                                       with_grad=True).items()}
    o, lse = fsa.forward(x["q"], x["k"], x["v"], alpha=1.0, w=8, R=1 << 16, scale=0.125)
    out = [torch.full(x["q"].shape, 7.0, dtype=torch.float32, device=dev()) for _ in range(3)]
    st = noalloc(x["q"], x["k"], x["v"], o, lse, x["do"], *out, 1.0, 8, 1 << 16)
    assert st == fsa.FSA_E_CAPACITY
    assert b"scratch" in fsa.library().fsa_last_error()
    torch.cuda.synchronize()
    assert all(bool((t == 7.0).all()) for t in out)  # nothing ran
    case(221, (1, 8, 32768, 64), torch.bfloat16, 1.0, 64, 1024)
