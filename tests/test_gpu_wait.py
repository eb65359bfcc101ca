"""The one-launch backward's bounded waits, seen from the host.

The one-launch backward (B * H a multiple of 8) lets its dK/dV workgroups wait for the
dQ workgroups' per-tile tokens. Each wait is bounded; a wait that gives up stores NaN
gradients and writes the launch's token into the workspace's status word, which
fsa_wait_status reads. Here the give-up is forced from the host
(fsa_debug_force_wait_timeout: the waits look for a value no workgroup publishes and
stop after a few polls), so every kernel still exits normally; the tests check that
the call then reports the failure, that a normal call reports none, and that the next
normal call on the same workspace is correct again."""
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


@pytest.fixture
def forced():
    fsa.debug_force_wait_timeout(True)
    try:
        yield
    finally:
        fsa.debug_force_wait_timeout(False)


def inputs(seed, shape):
    return {k: v.to(dev()) for k, v in synth.layer_inputs(seed, 0, shape, torch.bfloat16, with_grad=True).items()}


@pytest.mark.parametrize("w", [64, 16], ids=["bf16-slots", "fp32-slots"])
def test_static_give_up_is_reported(w):
    x = inputs(120, (2, 4, 500, 64))
    kw = dict(alpha=1.1, w=w, R=1024, scale=0.125)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], **kw)
    need = fsa.workspace_bytes(torch.bfloat16, 2, 4, 500, alpha=1.1, w=w, R=1024)
    ws = torch.empty(need // 4 + 1, dtype=torch.int32, device=dev())
    note(f"static backward w={w}: normal call, then a forced give-up, then a normal call")
    g0 = fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], pair_ws=ws, out_dtype=torch.float32, **kw)
    assert not fsa.wait_status("backward", x["q"], ws, alpha=1.1, w=w, R=1024)
    assert all(bool(torch.isfinite(t).all()) for t in g0)
    fsa.debug_force_wait_timeout(True)
    try:
        g1 = fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], pair_ws=ws, out_dtype=torch.float32, **kw)
        gave_up = fsa.wait_status("backward", x["q"], ws, alpha=1.1, w=w, R=1024)
    finally:
        fsa.debug_force_wait_timeout(False)
    assert gave_up
    # the dQ work never waits; the dK/dV work of every tile gave up and shows NaN
    assert torch.equal(g1[0], g0[0])
    assert bool(torch.isnan(g1[1]).all()) and bool(torch.isnan(g1[2]).all())
    g2 = fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], pair_ws=ws, out_dtype=torch.float32, **kw)
    assert not fsa.wait_status("backward", x["q"], ws, alpha=1.1, w=w, R=1024)
    for a, b in zip(g0, g2):
        assert torch.equal(a, b)


def test_two_kernel_shapes_have_no_waits(forced):
    x = inputs(121, (1, 3, 300, 64))
    kw = dict(alpha=1.0, w=64, R=1024, scale=0.125)
    o, lse = fsa.forward(x["q"], x["k"], x["v"], **kw)
    need = fsa.workspace_bytes(torch.bfloat16, 1, 3, 300, alpha=1.0, w=64, R=1024)
    ws = torch.empty(need // 4 + 1, dtype=torch.int32, device=dev())
    g = fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], pair_ws=ws, **kw)
    assert not fsa.wait_status("backward", x["q"], ws, alpha=1.0, w=64, R=1024)
    assert all(bool(torch.isfinite(t).all()) for t in g)


def test_frac_give_up_is_reported():
    x = inputs(122, (1, 8, 400, 64))
    kw = dict(alpha=1.13, w=64, R=1024, scale=0.125)
    o, lse = fsa.frac_forward(x["q"], x["k"], x["v"], **kw)
    need = fsa.frac_workspace_bytes(torch.bfloat16, 1, 8, 400, alpha=1.13, w=64, R=1024)
    ws = torch.empty(need // 4 + 1, dtype=torch.int32, device=dev())
    g0 = fsa.frac_backward(x["q"], x["k"], x["v"], o, lse, x["do"], ws=ws, **kw)
    assert not fsa.wait_status("frac_backward", x["q"], ws, alpha=1.13, w=64, R=1024)
    fsa.debug_force_wait_timeout(True)
    try:
        g1 = fsa.frac_backward(x["q"], x["k"], x["v"], o, lse, x["do"], ws=ws, **kw)
        gave_up = fsa.wait_status("frac_backward", x["q"], ws, alpha=1.13, w=64, R=1024)
    finally:
        fsa.debug_force_wait_timeout(False)
    assert gave_up
    assert bool(torch.isnan(g1[1]).all()) and bool(torch.isnan(g1[3]).all())
    g2 = fsa.frac_backward(x["q"], x["k"], x["v"], o, lse, x["do"], ws=ws, **kw)
    assert not fsa.wait_status("frac_backward", x["q"], ws, alpha=1.13, w=64, R=1024)
    for a, b in zip(g0, g2):
        assert torch.equal(a, b)


def test_rope_give_up_is_reported():
    x = inputs(123, (2, 4, 300, 64))
    table = fsa.rope_table(300, device=dev())
    kw = dict(alpha=1.2, w=64, R=1024, scale=0.125)
    o, lse = fsa.rope_forward(x["q"], x["k"], x["v"], table, **kw)
    need = fsa.rope_workspace_bytes(torch.bfloat16, 2, 4, 300, alpha=1.2, w=64, R=1024)[1]
    ws = torch.empty(need // 4 + 1, dtype=torch.int32, device=dev())
    fsa.debug_force_wait_timeout(True)
    try:
        g = fsa.rope_backward(x["q"], x["k"], x["v"], table, o, lse, x["do"], ws=ws, **kw)
        gave_up = fsa.wait_status("rope_backward", x["q"], ws, alpha=1.2, w=64, R=1024)
    finally:
        fsa.debug_force_wait_timeout(False)
    assert gave_up and bool(torch.isnan(g[1].float()).all())
    fsa.rope_backward(x["q"], x["k"], x["v"], table, o, lse, x["do"], ws=ws, **kw)
    assert not fsa.wait_status("rope_backward", x["q"], ws, alpha=1.2, w=64, R=1024)


def test_rope_forward_give_up_is_reported():
    # B * H = 8: the rotary forward rotates K in the kernel; tiles read the rotated rows of
    # earlier tiles after waiting for their tokens. Tile 0 of each head waits for none.
    x = inputs(124, (2, 4, 300, 64))
    table = fsa.rope_table(300, device=dev())
    kw = dict(alpha=1.2, w=64, R=1024, scale=0.125)
    need = fsa.rope_workspace_bytes(torch.bfloat16, 2, 4, 300, alpha=1.2, w=64, R=1024)[0]
    ws = torch.empty(need // 4 + 1, dtype=torch.int32, device=dev())
    o0, l0 = fsa.rope_forward(x["q"], x["k"], x["v"], table, ws=ws, **kw)
    assert not fsa.wait_status("rope_forward", x["q"], ws, alpha=1.2, w=64, R=1024)
    fsa.debug_force_wait_timeout(True)
    try:
        o1, l1 = fsa.rope_forward(x["q"], x["k"], x["v"], table, ws=ws, **kw)
        gave_up = fsa.wait_status("rope_forward", x["q"], ws, alpha=1.2, w=64, R=1024)
    finally:
        fsa.debug_force_wait_timeout(False)
    note(f"rope forward forced give-up reported: {gave_up}")
    assert gave_up
    assert torch.equal(o1[:, :, :64], o0[:, :, :64]) and torch.equal(l1[:, :, :64], l0[:, :, :64])
    assert bool(torch.isnan(o1[:, :, 64:].float()).all()) and bool(torch.isnan(l1[:, :, 64:]).all())
    o2, l2 = fsa.rope_forward(x["q"], x["k"], x["v"], table, ws=ws, **kw)
    assert not fsa.wait_status("rope_forward", x["q"], ws, alpha=1.2, w=64, R=1024)
    assert torch.equal(o2, o0) and torch.equal(l2, l0)
