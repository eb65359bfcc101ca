"""The rounding allowance used by the rotary GPU tests (rope_rounding), checked on the
CPU: any rotation within the fp32 error bound of the exact one stores, element by
element, a value within the flagged range, and rounds apart from the stored rows only
at flagged elements."""
import numpy as np
import pytest

import oracle
import rope_rounding as RR


@pytest.mark.parametrize("seed", range(3))
def test_rotations_within_the_bound_store_within_the_flagged_ranges(seed):
    r = np.random.default_rng(100 + seed)
    N = 300
    x = oracle.bf16_round(r.standard_normal((N, 64)) * r.choice([0.01, 1.0, 30.0], size=(N, 1)))
    y = oracle.rope_rotate(x)
    stored, amb = RR.ambiguous(x, slack=1.0)
    assert np.array_equal(stored, oracle.rope_store_bf16(x))
    lo, hi = stored.copy(), stored.copy()
    for i, ends in amb:
        assert ends and all(e != stored[i] for e in ends)
        lo[i] = min([stored[i]] + ends)
        hi[i] = max([stored[i]] + ends)
    bound = RR.rotation_bound(x, slack=1.0)
    moved = 0
    for t in range(200):
        u = r.uniform(-1.0, 1.0, size=x.shape)
        if t % 4 == 0:
            u = np.sign(u)  # the ends of the bound
        z = oracle.bf16_round(y + bound * u)
        assert np.all((z >= lo) & (z <= hi))
        moved += int(np.count_nonzero(z != stored))
    assert len(amb) > 0 and moved > 0


def test_cancelling_pairs_flag_ranges_of_several_values():
    # a pair whose rotation nearly cancels: the bound, relative to the pair, spans many
    # bf16 steps of the small result
    th = 1.0  # position 1, channel pair 0: angle 1 rad
    x = np.zeros((2, 64))
    x[1, 0], x[1, 1] = oracle.bf16_round(np.sin(th)), oracle.bf16_round(np.cos(th))
    y = oracle.rope_rotate(x)
    assert abs(y[1, 0]) < 1e-2 * (abs(x[1, 0]) + abs(x[1, 1]))
    _, amb = RR.ambiguous(x)
    assert any(i == (1, 0) for i, _ in amb)


def test_allowance_counts_every_flagged_element():
    r = np.random.default_rng(9)
    N = 90
    q, k = (oracle.bf16_round(r.standard_normal((N, 64))) for _ in range(2))
    v, do = (oracle.bf16_round(r.standard_normal((N, 64))) for _ in range(2))
    entries = [66.25, 80.5]
    o, lse = oracle.frac_forward(oracle.rope_store_bf16(q), oracle.rope_store_bf16(k), v, entries, 8, 0.125)
    allow, n = RR.entry_grad_allowance(q, k, v, do, entries, 8, 0.125, o, lse)
    assert n == len(RR.ambiguous(q)[1]) + len(RR.ambiguous(k)[1])
    assert allow.shape == (2,) and np.all(allow >= 0.0)
    assert n == 0 or np.any(allow > 0.0)
