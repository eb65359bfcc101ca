"""Allowance for checks of the learned-alpha entry gradient over rotated rows.

The rotary reading stores each rotated row as the exact rotation rounded once to
bfloat16 (oracle.rope_store_bf16). The library's rotation forms the same value in fp32
(fp32 cos/sin table, one product and one fused multiply-add) before that rounding, which
is within 2^-22 (|x_even| + |x_odd|) of the exact value y. Rounding is monotonic, so that
value stores as a bf16 value between those of y - bound and y + bound: the stored rows
agree except where that range holds more than one value (next to a rounding boundary,
or several values apart where the pair's two products nearly cancel). The entry
gradient (an fp32 sum checked to 1e-5 of its terms' absolute values when the inputs
agree) is then allowed, in addition, the sum over those elements of how far the oracle's
entry gradient moves when that one element takes the farther end of its range. Used by
the rotary GPU tests only; plain numpy over the oracle's functions."""
import numpy as np

import oracle


def rotation_bound(x, slack: float = 2.0):
    """Per element of the rotated rows of x [N, d]: slack * 2^-22 (|x_even| + |x_odd|) of
    its channel pair, the distance within which an fp32 rotation lands."""
    pair = np.abs(x[:, 0::2]) + np.abs(x[:, 1::2])
    return slack * 2.0 ** -22 * np.repeat(pair, 2, axis=1)


def ambiguous(x, base: float = 10000.0, slack: float = 2.0):
    """Rows x [N, d] (unrotated, exact): the stored rows r and, for every element whose
    range of stored values holds more than r, (index, [the range's ends other than r])."""
    y = oracle.rope_rotate(x, base)
    r = oracle.rope_store_bf16(x, base)
    b = rotation_bound(x, slack)
    lo, hi = oracle.bf16_round(y - b), oracle.bf16_round(y + b)
    idx = np.argwhere((lo != r) | (hi != r))
    return r, [(tuple(i), [e for e in {lo[tuple(i)], hi[tuple(i)]} if e != r[tuple(i)]]) for i in idx]


def entry_grad_allowance(q, k, v, do, entries, w, scale, o, lse, base: float = 10000.0):
    """Per entry: sum over the ambiguous elements of the rotated q and k rows of one head
    of the largest |change of the oracle's entry gradient| when that element takes an end
    of its range (o and lse given, as the backward receives them). Also returns the count
    of such elements."""
    qr, amb_q = ambiguous(q, base)
    kr, amb_k = ambiguous(k, base)
    dd0 = oracle.frac_backward(qr, kr, v, do, entries, w, scale, o=o, lse=lse)[3]
    total = np.zeros_like(dd0)
    for which, amb in ((0, amb_q), (1, amb_k)):
        for i, ends in amb:
            worst = np.zeros_like(dd0)
            for val in ends:
                a, b = qr.copy(), kr.copy()
                (a if which == 0 else b)[i] = val
                worst = np.maximum(worst, np.abs(oracle.frac_backward(a, b, v, do, entries, w, scale, o=o, lse=lse)[3] - dd0))
            total += worst
    return total, len(amb_q) + len(amb_k)
