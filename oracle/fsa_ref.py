"""Plain fp64 CPU oracle for Fibonacci-offset sparse attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this
module; only the test suite, the package smoke check and the benchmark's
CPU-baseline leg use it. It shares no code, tables or constants with the HIP
library: it re-derives everything from the pages in the plainest form.

Pages cited (titles as published):
  [EXPL-pt] "Depth-Staggered Fibonacci Spacing for Sparse Attention: Static
            Schedules Beat Learned Dilation and Extrapolate Where Dense
            Attention Fails", gist.science explainer of C. A. Capps' paper,
            Portuguese edition.
  [EXPL-fr] the same explainer, French edition (same sections, translated).
  [SUMM-zh] "深度解读：基于深度交错斐波那契间隔的稀疏注意力机制" (aimsg.uk
            summary of the same paper), section "核心内容".

What the pages fix:
  * [EXPL-pt] Metodologia / Arquitetura e Mecanismo de Atenção, item
    "Conjunto Atendido": query i attends a dense local window of size W plus
    sparse offsets from the Fibonacci list 1, 2, 3, 5, ..., 987.
  * same section, item "Escalonamento": every offset f_k is scaled by a
    per-layer scalar, d_k = alpha * f_k, with alpha restricted to [0.5, 1.5].
  * [EXPL-pt] Variáveis Experimentais: fixed schedule alpha = 1 for all layers;
    static linear stagger rising from 0.5 at layer 0 to 1.5 at layer 15.
  * [EXPL-pt] Controles: a reach-matched power-of-2 (log-sparse) base; a dense
    baseline with the same architecture.
  * [EXPL-pt] Principais Contribuições e Resultados, item 2 ("Eficiência"):
    static schedules execute as a boolean mask, so the offsets are integers and
    each key is attended at most once.

Readings taken where the pages leave a step open (all switchable here only):
  * rounding of alpha*F: round half to even on the fp64 product (the half-away
    variant exists for tests that show which tables the choice moves);
  * reach R caps the base value (F < R, exclusive), before scaling;
  * the window holds offsets 0..w-1 (self included); sparse offsets below w
    merge into it; duplicates collapse (set semantics);
  * keys before the sequence start are dropped (no padding, no wrap);
  * one softmax over window and sparse offsets together;
  * the backward pass is the textbook softmax-attention gradient restricted to
    the mask.

Floating point: every array is converted to float64 on entry.
"""
from __future__ import annotations

import math

import numpy as np

# ----------------------------------------------------------------------------
# Offset tables
# ----------------------------------------------------------------------------


def fibonacci_base(R: int) -> list[int]:
    """Distinct Fibonacci numbers F < R, starting 1, 2, 3, 5, ...

    [EXPL-pt] Metodologia / Arquitetura, "Conjunto Atendido": the printed list
    starts 1, 2, 3, 5 (no repeated 1) and ends at 987 when the reach is 1024.
    Recurrence F_1 = 1, F_2 = 2, F_{k+1} = F_k + F_{k-1}; R is exclusive.
    """
    out = []
    a, b = 1, 2
    while a < R:
        out.append(a)
        a, b = b, a + b
    return out


def pow2_base(R: int) -> list[int]:
    """Powers of two 2^k < R, k >= 0.

    [EXPL-pt] Controles: a reach-matched power-of-2 (log-sparse) base.
    """
    out = []
    p = 1
    while p < R:
        out.append(p)
        p *= 2
    return out


def round_half_even(x: float) -> int:
    """Round a finite double to the nearest integer, ties to the even one.

    Written out so that a reader can check it: f = floor(x), r = x - f is exact
    for doubles of this magnitude; r > 1/2 rounds up, r < 1/2 rounds down, and
    r == 1/2 picks whichever of f, f+1 is even.
    """
    f = math.floor(x)
    r = x - f
    if r > 0.5:
        return int(f) + 1
    if r < 0.5:
        return int(f)
    return int(f) if int(f) % 2 == 0 else int(f) + 1


def round_half_away(x: float) -> int:
    """Alternative reading: ties away from zero (x > 0 here)."""
    f = math.floor(x)
    r = x - f
    return int(f) + 1 if r >= 0.5 else int(f)


def offset_table(base: str, alpha: float, w: int, R: int,
                 rounding: str = "even") -> list[int]:
    """Sparse offsets T for one layer: sorted unique round(alpha*F) that are >= w.

    [EXPL-pt] Metodologia / Arquitetura, items "Conjunto Atendido" and
    "Escalonamento": d_k = alpha * f_k over the base list. Values below w fall
    inside the dense window and are dropped from T; T does not depend on N.
    """
    if base == "fib":
        fs = fibonacci_base(R)
    elif base == "pow2":
        fs = pow2_base(R)
    else:
        raise ValueError(f"unknown base {base!r}")
    rnd = round_half_even if rounding == "even" else round_half_away
    alpha = float(alpha)
    scaled = [rnd(alpha * float(f)) for f in fs]
    return sorted({o for o in scaled if o >= w})


def attended_offsets(T: list[int], w: int) -> list[int]:
    """Full offset set O = {0, ..., w-1} union T (sorted, unique)."""
    return sorted(set(range(w)) | set(int(o) for o in T))


def stagger_alpha(layer: int, n_layers: int = 16) -> float:
    """Static linear stagger: alpha rises linearly from 0.5 at layer 0 to 1.5
    at the last layer ([EXPL-pt] Variáveis Experimentais, "Escalonado
    (Linear)"). Computed as 0.5 + layer / (n_layers - 1) in fp64."""
    return 0.5 + layer / float(n_layers - 1)


def coprime_layer(layer: int, n_layers: int = 16) -> int:
    """Coprime reassignment layer -> 7*layer mod L ([EXPL-pt] Variáveis
    Experimentais, "Escalonado (Coprimo/HDC)")."""
    return (7 * layer) % n_layers


# ----------------------------------------------------------------------------
# Attention: forward, backward, dense baseline
# ----------------------------------------------------------------------------


def _scores(q, k, offs, scale):
    """S[..., i, m] = scale * <q_i, k_{i - offs[m]}>, -inf where i - offs[m] < 0."""
    N = q.shape[-2]
    S = np.full(q.shape[:-1] + (len(offs),), -np.inf)
    for m, o in enumerate(offs):
        if o < N:
            S[..., o:, m] = scale * np.sum(q[..., o:, :] * k[..., : N - o, :], axis=-1)
    return S


def _softmax_rows(S):
    """Two-pass softmax over the last axis; returns P, row max, row sum."""
    mx = np.max(S, axis=-1, keepdims=True)
    e = np.exp(S - mx)
    l = np.sum(e, axis=-1, keepdims=True)
    return e / l, mx[..., 0], l[..., 0]


def sparse_probabilities(q, k, T, w, scale):
    """P[..., i, m] over the offset list O = {0..w-1} u T, plus row max/sum."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    offs = attended_offsets(T, w)
    S = _scores(q, k, offs, scale)
    P, mx, l = _softmax_rows(S)
    return offs, P, mx, l


def sparse_forward(q, k, v, T, w, scale):
    """o_i = sum_{j in J(i)} P_ij v_j and LSE_i = m_i + ln l_i, where
    J(i) = {i - o : o in {0..w-1} u T, o <= i}.

    Layout: [..., N, d]; returns (o [..., N, d], lse [..., N]) in float64.
    [EXPL-pt] Metodologia / Arquitetura, "Conjunto Atendido" (the attended set)
    and Principais Contribuições §2 (a single boolean mask, so one softmax).
    """
    v = np.asarray(v, dtype=np.float64)
    offs, P, mx, l = sparse_probabilities(q, k, T, w, scale)
    N = v.shape[-2]
    o = np.zeros(v.shape)
    for m, off in enumerate(offs):
        if off < N:
            o[..., off:, :] += P[..., off:, m : m + 1] * v[..., : N - off, :]
    return o, mx + np.log(l)


def sparse_backward(q, k, v, dout, T, w, scale, o=None, lse=None):
    """Gradients of sum(dout * o) with respect to q, k, v.

    Textbook softmax-attention gradient restricted to the mask:
      D_i = <dO_i, o_i>, dP_ij = <dO_i, v_j>, dS_ij = P_ij (dP_ij - D_i),
      dQ_i = scale sum_j dS_ij k_j, dK_j = scale sum_i dS_ij q_i,
      dV_j = sum_i P_ij dO_i, all sums over pairs with j in J(i).
    The pages describe training through this mask ([EXPL-pt] Metodologia) but
    print no gradient, so this is the plain derivative of the forward above.
    o and lse, when given, are the forward outputs the backward is handed (for
    instance rounded to a storage type): then P_ij = exp(s_ij - lse_i) and
    D_i = <dout_i, o_i>, the same formula with those inputs. Otherwise both come
    from this module's exact forward.
    Returns (dq, dk, dv) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    offs, P, _, _ = sparse_probabilities(q, k, T, w, scale)
    if lse is not None:
        P = np.exp(_scores(q, k, offs, scale) - np.asarray(lse, dtype=np.float64)[..., None])
    if o is None:
        o, _ = sparse_forward(q, k, v, T, w, scale)
    N = q.shape[-2]
    D = np.sum(dout * np.asarray(o, dtype=np.float64), axis=-1)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for m, off in enumerate(offs):
        if off >= N:
            continue
        qi, doi = q[..., off:, :], dout[..., off:, :]
        kj, vj = k[..., : N - off, :], v[..., : N - off, :]
        p = P[..., off:, m]
        dp = np.sum(doi * vj, axis=-1)
        ds = p * (dp - D[..., off:])
        dq[..., off:, :] += scale * ds[..., None] * kj
        dk[..., : N - off, :] += scale * ds[..., None] * qi
        dv[..., : N - off, :] += p[..., None] * doi
    return dq, dk, dv


def dense_forward(q, k, v, scale):
    """Dense causal baseline: o = softmax(scale * q k^T masked to j <= i) v.

    [EXPL-pt] Controles: dense attention with the same architecture.
    Full N x N matrix; fine for the sizes the tests use.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N = q.shape[-2]
    S = scale * (q @ np.swapaxes(k, -1, -2))
    future = np.triu(np.ones((N, N), dtype=bool), k=1)
    S = np.where(future, -np.inf, S)
    P, mx, l = _softmax_rows(S)
    return P @ v, mx + np.log(l)


def dense_forward_rows(q, k, v, scale, rows):
    """Dense causal output for selected query rows only (for large N checks).

    rows: 1-D integer array of query indices. Returns (o [..., len(rows), d],
    lse [..., len(rows)]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    outs, lses = [], []
    for i in rows:
        i = int(i)
        s = scale * np.sum(q[..., i : i + 1, :] * k[..., : i + 1, :], axis=-1)
        mx = np.max(s, axis=-1, keepdims=True)
        e = np.exp(s - mx)
        l = np.sum(e, axis=-1, keepdims=True)
        outs.append(np.sum((e / l)[..., None] * v[..., : i + 1, :], axis=-2))
        lses.append(mx[..., 0] + np.log(l[..., 0]))
    return np.stack(outs, axis=-2), np.stack(lses, axis=-1)


# ----------------------------------------------------------------------------
# Row-sampled forms of the same definitions (for full-size checks)
# ----------------------------------------------------------------------------


def _row_keys(i, offs):
    """Key indices J(i) = {i - o : o in offs, o <= i} (ascending offset order)."""
    return [i - o for o in offs if o <= i]


def sparse_forward_rows(q, k, v, T, w, scale, rows):
    """o_i and LSE_i of sparse_forward for the given query rows, one by one.

    q, k, v: [..., N, d]. Returns (o [..., len(rows), d], lse [..., len(rows)]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    offs = attended_offsets(T, w)
    outs, lses = [], []
    for i in rows:
        js = _row_keys(int(i), offs)
        s = scale * np.sum(q[..., int(i) : int(i) + 1, :] * k[..., js, :], axis=-1)
        mx = np.max(s, axis=-1, keepdims=True)
        e = np.exp(s - mx)
        l = np.sum(e, axis=-1, keepdims=True)
        outs.append(np.sum((e / l)[..., None] * v[..., js, :], axis=-2))
        lses.append(mx[..., 0] + np.log(l[..., 0]))
    return np.stack(outs, axis=-2), np.stack(lses, axis=-1)


def sparse_backward_rows(q, k, v, dout, T, w, scale, rows):
    """dQ_r, dK_r, dV_r of sparse_backward for the given rows r, one by one.

    dQ_r sums over the keys row r attends; dK_r and dV_r sum over the queries
    i = r + o (o in O, i < N) that attend key r. Each needed P_ij comes from
    that query's own softmax (its LSE and o_i), recomputed per row.
    Returns (dq, dk, dv), each [..., len(rows), d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    N = q.shape[-2]
    offs = attended_offsets(T, w)

    cache = {}

    def row_stats(i):
        # (keys, P over those keys, D_i) for query row i
        if i not in cache:
            js = _row_keys(i, offs)
            s = scale * np.sum(q[..., i : i + 1, :] * k[..., js, :], axis=-1)
            mx = np.max(s, axis=-1, keepdims=True)
            e = np.exp(s - mx)
            p = e / np.sum(e, axis=-1, keepdims=True)
            o_i = np.sum(p[..., None] * v[..., js, :], axis=-2)
            D = np.sum(dout[..., i, :] * o_i, axis=-1)
            cache[i] = (js, p, D)
        return cache[i]

    dqs, dks, dvs = [], [], []
    for r in rows:
        r = int(r)
        js, p, D = row_stats(r)
        dp = np.sum(dout[..., r : r + 1, :] * v[..., js, :], axis=-1)
        ds = p * (dp - D[..., None])
        dqs.append(scale * np.sum(ds[..., None] * k[..., js, :], axis=-2))
        dk_r = np.zeros(q.shape[:-2] + (q.shape[-1],))
        dv_r = np.zeros(q.shape[:-2] + (q.shape[-1],))
        for o in offs:
            i = r + o
            if i >= N:
                continue
            jsi, pi, Di = row_stats(i)
            col = jsi.index(r)
            p_ir = pi[..., col]
            dp_ir = np.sum(dout[..., i, :] * v[..., r, :], axis=-1)
            ds_ir = p_ir * (dp_ir - Di)
            dk_r += scale * ds_ir[..., None] * q[..., i, :]
            dv_r += p_ir[..., None] * dout[..., i, :]
        dks.append(dk_r)
        dvs.append(dv_r)
    return np.stack(dqs, axis=-2), np.stack(dks, axis=-2), np.stack(dvs, axis=-2)


# ----------------------------------------------------------------------------
# Fractional offsets: the learned-alpha variant
# ----------------------------------------------------------------------------
#
# [EXPL-pt] Metodologia / Arquitetura, item "Implementação": when alpha is a
# learned parameter the targets d_k = alpha * f_k are not integers, and the model
# interpolates linearly between key/value rows so that a gradient reaches alpha.
# [EXPL-pt] Variáveis Experimentais, "Aprendido": one free parameter per layer,
# started at alpha = 1. [EXPL-pt] Principais Contribuições §2 ("Eficiência"):
# this variant ran as an unfused interpolated gather.
#
# Readings taken where the pages leave a step open:
#   * d_k = alpha * f_k is one fp64 product and is not rounded; the entry is kept
#     when d_k >= w (the same threshold as the static table);
#   * the virtual key of query i for entry k sits at position i - d_k: with
#     a = floor(d_k) and phi = d_k - a it is (1 - phi) * row(i - a) +
#     phi * row(i - a - 1), for keys and values alike (the two rows around that
#     position, weighted by closeness);
#   * the entry exists for query i when i - d_k >= 0 (no row before the start);
#   * every entry is its own column of the one softmax (distinct f give distinct
#     d; entries are not merged with the window or with each other);
#   * at an integer d_k the derivative is the one-sided one of the piece
#     [a, a + 1), k(i - a - 1) - k(i - a) (what a floor-based interpolation
#     differentiates to); a query without the row i - a - 1 contributes none;
#   * d(loss)/d(alpha) = sum_k f_k d(loss)/d(d_k), summed over batch, heads and
#     rows, since alpha is one scalar per layer.


def frac_offset_table(base: str, alpha: float, w: int, R: int) -> list[tuple[float, int]]:
    """Entries (d_k, f_k) of the learned-alpha variant: d_k = alpha * f_k in fp64,
    kept when d_k >= w, in increasing order of d_k."""
    if base == "fib":
        fs = fibonacci_base(R)
    elif base == "pow2":
        fs = pow2_base(R)
    else:
        raise ValueError(f"unknown base {base!r}")
    alpha = float(alpha)
    return sorted((alpha * float(f), f) for f in fs if alpha * float(f) >= w)


def _split(d: float) -> tuple[int, float, int]:
    """a = floor(d), phi = d - a, and the first query row i0 = ceil(d) that has the entry."""
    a = math.floor(d)
    phi = d - a
    return int(a), phi, int(a) if phi == 0.0 else int(a) + 1


def _virtual_rows(x, d: float):
    """Rows (1 - phi) x[i - a] + phi x[i - a - 1] for i = i0 .. N-1, or None if i0 >= N."""
    N = x.shape[-2]
    a, phi, i0 = _split(d)
    if i0 >= N:
        return i0, None
    near = x[..., i0 - a : N - a, :]
    if phi == 0.0:
        return i0, near.copy()
    far = x[..., i0 - a - 1 : N - a - 1, :]
    return i0, (1.0 - phi) * near + phi * far


def _frac_scores(q, k, entries, w, scale):
    """Scores over columns [window offsets 0..w-1, then one column per entry], -inf where absent."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    N = q.shape[-2]
    S = np.full(q.shape[:-1] + (w + len(entries),), -np.inf)
    for o in range(min(w, N)):
        S[..., o:, o] = scale * np.sum(q[..., o:, :] * k[..., : N - o, :], axis=-1)
    for m, d in enumerate(entries):
        i0, kt = _virtual_rows(k, d)
        if kt is not None:
            S[..., i0:, w + m] = scale * np.sum(q[..., i0:, :] * kt, axis=-1)
    return S


def frac_probabilities(q, k, entries, w, scale):
    """P over columns [window offsets 0..w-1, then one column per entry], row max, row sum."""
    return _softmax_rows(_frac_scores(q, k, entries, w, scale))


def frac_forward(q, k, v, entries, w, scale):
    """Forward of the learned-alpha variant: one softmax over the window keys and the
    interpolated entry keys, output the same mix of window and interpolated values.

    entries: the d_k of frac_offset_table (floats). Returns (o, lse) in float64.
    """
    v = np.asarray(v, dtype=np.float64)
    P, mx, l = frac_probabilities(q, k, entries, w, scale)
    N = v.shape[-2]
    o = np.zeros(v.shape)
    for off in range(min(w, N)):
        o[..., off:, :] += P[..., off:, off : off + 1] * v[..., : N - off, :]
    for m, d in enumerate(entries):
        i0, vt = _virtual_rows(v, d)
        if vt is not None:
            o[..., i0:, :] += P[..., i0:, w + m : w + m + 1] * vt
    return o, mx + np.log(l)


def frac_backward(q, k, v, dout, entries, w, scale, o=None, lse=None):
    """Gradients of sum(dout * o) for the learned-alpha variant.

    Returns (dq, dk, dv, dd) where dd[m] is the derivative with respect to d_m,
    summed over every leading index and row; d(loss)/d(alpha) is
    sum_m f_m dd[m]. The score and value paths are the textbook softmax-attention
    gradient; an interpolated row passes its gradient to its two source rows with
    the weights (1 - phi) and phi.

    o and lse, when given, are the forward outputs the backward is handed (for
    instance rounded to a storage type): then P_ij = exp(s_ij - lse_i) and
    D_i = <dout_i, o_i>, the same formula with those inputs. Otherwise both
    come from this module's exact forward.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    N = q.shape[-2]
    if lse is None:
        P, _, _ = frac_probabilities(q, k, entries, w, scale)
    else:
        P = np.exp(_frac_scores(q, k, entries, w, scale) - np.asarray(lse, dtype=np.float64)[..., None])
    if o is None:
        o, _ = frac_forward(q, k, v, entries, w, scale)
    D = np.sum(dout * np.asarray(o, dtype=np.float64), axis=-1)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for off in range(min(w, N)):
        p = P[..., off:, off]
        dp = np.sum(dout[..., off:, :] * v[..., : N - off, :], axis=-1)
        ds = p * (dp - D[..., off:])
        dq[..., off:, :] += scale * ds[..., None] * k[..., : N - off, :]
        dk[..., : N - off, :] += scale * ds[..., None] * q[..., off:, :]
        dv[..., : N - off, :] += p[..., None] * dout[..., off:, :]
    dd = np.zeros(len(entries))
    for m, d in enumerate(entries):
        a, phi, i0 = _split(d)
        if i0 >= N:
            continue
        _, kt = _virtual_rows(k, d)
        _, vt = _virtual_rows(v, d)
        p = P[..., i0:, w + m]
        dp = np.sum(dout[..., i0:, :] * vt, axis=-1)
        ds = p * (dp - D[..., i0:])
        dq[..., i0:, :] += scale * ds[..., None] * kt
        gk = scale * ds[..., None] * q[..., i0:, :]  # gradient reaching the virtual key
        gv = p[..., None] * dout[..., i0:, :]        # and the virtual value
        dk[..., i0 - a : N - a, :] += (1.0 - phi) * gk
        dv[..., i0 - a : N - a, :] += (1.0 - phi) * gv
        if phi != 0.0:
            dk[..., i0 - a - 1 : N - a - 1, :] += phi * gk
            dv[..., i0 - a - 1 : N - a - 1, :] += phi * gv
        # d/d(d_m) of the virtual rows: row(i - a - 1) - row(i - a), rows i >= a + 1
        s0 = max(i0, a + 1)
        if s0 < N:
            c = s0 - i0
            dkr = k[..., s0 - a - 1 : N - a - 1, :] - k[..., s0 - a : N - a, :]
            dvr = v[..., s0 - a - 1 : N - a - 1, :] - v[..., s0 - a : N - a, :]
            dd[m] = np.sum(np.sum(gk[..., c:, :] * dkr, axis=-1)) + np.sum(np.sum(gv[..., c:, :] * dvr, axis=-1))
    return dq, dk, dv, dd


def frac_alpha_grad(dd, fs) -> float:
    """d(loss)/d(alpha) = sum_m f_m dd[m] (alpha scales every d_m = alpha f_m)."""
    return float(sum(float(f) * float(x) for f, x in zip(fs, dd)))


def _frac_row_sources(i: int, entries, w: int):
    """Attended columns of query row i as lists of (key row, weight) pairs:
    window keys first, then one virtual key per entry present at row i."""
    cols = [[(i - o, 1.0)] for o in range(w) if o <= i]
    for d in entries:
        a, phi, i0 = _split(d)
        if i < i0:
            continue
        cols.append([(i - a, 1.0)] if phi == 0.0 else [(i - a, 1.0 - phi), (i - a - 1, phi)])
    return cols


def frac_forward_rows(q, k, v, entries, w, scale, rows):
    """o_i and LSE_i of frac_forward for the given query rows, one by one."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    outs, lses = [], []
    for i in rows:
        i = int(i)
        cols = _frac_row_sources(i, entries, w)
        kt = np.stack([sum(c * k[..., j, :] for j, c in col) for col in cols], axis=-2)
        vt = np.stack([sum(c * v[..., j, :] for j, c in col) for col in cols], axis=-2)
        s = scale * np.sum(q[..., i : i + 1, :] * kt, axis=-1)
        mx = np.max(s, axis=-1, keepdims=True)
        e = np.exp(s - mx)
        lsum = np.sum(e, axis=-1, keepdims=True)
        outs.append(np.sum((e / lsum)[..., None] * vt, axis=-2))
        lses.append(mx[..., 0] + np.log(lsum[..., 0]))
    return np.stack(outs, axis=-2), np.stack(lses, axis=-1)


def frac_backward_rows(q, k, v, dout, entries, w, scale, rows):
    """dQ_r, dK_r, dV_r of frac_backward for the given rows r, one by one.

    dK_r and dV_r collect, from every query i and column whose key mixes row r,
    that column's gradient times row r's weight in the mix. Returns (dq, dk, dv),
    each [..., len(rows), d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    N = q.shape[-2]
    cache = {}

    def row_stats(i):
        # (columns, virtual keys, virtual values, P, dS) of query row i
        if i not in cache:
            cols = _frac_row_sources(i, entries, w)
            kt = np.stack([sum(c * k[..., j, :] for j, c in col) for col in cols], axis=-2)
            vt = np.stack([sum(c * v[..., j, :] for j, c in col) for col in cols], axis=-2)
            s = scale * np.sum(q[..., i : i + 1, :] * kt, axis=-1)
            e = np.exp(s - np.max(s, axis=-1, keepdims=True))
            p = e / np.sum(e, axis=-1, keepdims=True)
            o_i = np.sum(p[..., None] * vt, axis=-2)
            D = np.sum(dout[..., i, :] * o_i, axis=-1)
            dp = np.sum(dout[..., i : i + 1, :] * vt, axis=-1)
            cache[i] = (cols, kt, p, p * (dp - D[..., None]))
        return cache[i]

    # queries whose columns can mix key row r: r + o (window), r + a and r + a + 1
    reach = set(range(w))
    for d in entries:
        a, _, _ = _split(d)
        reach.update((a, a + 1))
    dqs, dks, dvs = [], [], []
    for r in rows:
        r = int(r)
        _, kt, _, ds = row_stats(r)
        dqs.append(scale * np.sum(ds[..., None] * kt, axis=-2))
        dk_r = np.zeros(q.shape[:-2] + (q.shape[-1],))
        dv_r = np.zeros(q.shape[:-2] + (q.shape[-1],))
        for off in sorted(reach):
            i = r + off
            if i >= N:
                continue
            cols, _, p, dsi = row_stats(i)
            for m, col in enumerate(cols):
                for j, c in col:
                    if j == r:
                        dk_r += c * scale * dsi[..., m : m + 1] * q[..., i, :]
                        dv_r += c * p[..., m : m + 1] * dout[..., i, :]
        dks.append(dk_r)
        dvs.append(dv_r)
    return np.stack(dqs, axis=-2), np.stack(dks, axis=-2), np.stack(dvs, axis=-2)


# ----------------------------------------------------------------------------
# Rotary position embedding applied before the attention
# ----------------------------------------------------------------------------
#
# [EXPL-pt] Metodologia / Arquitetura, item "Implementação": rotary position
# embeddings are applied to queries and keys before the rows are gathered;
# [EXPL-pt] Limitações: the models use vanilla RoPE without scaling. The pages give
# no formula; the readings here are the original rotary formulation:
#   * channel pairs (2m, 2m + 1), m = 0 .. d/2 - 1, with frequency
#     theta_m = base^(-2m/d), base = 10000 (no scaling);
#   * the position of row i is i, for queries and keys alike;
#   * pair m of a row at position p is rotated by the angle p * theta_m;
#   * values are not rotated; the backward returns gradients with respect to the
#     unrotated Q and K.
# The rotated rows are handed to the attention in the input's storage type, as a
# separate rotation step would store them (rope_store_bf16): the exact rotation
# (fp64 cos and sin of the fp64 angle) rounded once to bfloat16, nearest with ties to
# even. A library that computes the rotation in fp32 before that rounding may land
# one bf16 step away from it where the exact value sits next to a rounding boundary.


def rope_angles(n_pos: int, d: int, base: float = 10000.0):
    """angle[p, m] = p * base^(-2m/d) in fp64, shape [n_pos, d/2]."""
    m = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-2.0 * m / d)
    return np.arange(n_pos, dtype=np.float64)[:, None] * theta[None, :]


def rope_rotate(x, base: float = 10000.0, inverse: bool = False):
    """Rotates pair m of row p of x [..., N, d] by p * theta_m (by the negative angle
    when inverse, which is the transpose of the rotation), exactly in fp64."""
    x = np.asarray(x, dtype=np.float64)
    N, d = x.shape[-2], x.shape[-1]
    ang = rope_angles(N, d, base)
    c, s = np.cos(ang), np.sin(ang)
    if inverse:
        s = -s
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def rope_table_f32(n_pos: int, d: int, base: float = 10000.0):
    """[n_pos, d/2, 2] float32 table of (cos, sin) of p * theta_m: each value computed
    in fp64 with the C library's cos and sin (Python's math module) and rounded once."""
    out = np.empty((n_pos, d // 2, 2), dtype=np.float32)
    for m in range(d // 2):
        theta = base ** (-2.0 * m / d)
        for pos in range(n_pos):
            a = pos * theta
            out[pos, m, 0] = math.cos(a)
            out[pos, m, 1] = math.sin(a)
    return out


def bf16_round(x):
    """Rounds float64 values to the nearest bfloat16 value (8 significant bits, fp32's
    exponent range), ties to even, in one step from the fp64 value (no intermediate
    float32). Returns float64. Written out: x = m * 2^e with 1/2 <= |m| < 1, so
    m * 2^8 holds the 8 kept bits in its integer part; numpy's rint rounds that to
    nearest, ties to even, exactly in fp64. Below 2^-126 (bf16 subnormals) the quantum
    is fixed at 2^-133."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    normal = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    sub = np.ldexp(np.rint(np.ldexp(x, 133)), -133)
    return np.where(np.abs(x) < 2.0 ** -126, sub, normal)


def rope_store_bf16(x, base: float = 10000.0):
    """Rotated rows of x [..., N, d] as a rotation step that stores bf16 hands them to the
    attention: the exact fp64 rotation (rope_rotate) rounded once to bfloat16
    (bf16_round). Returns the bf16 values as float64."""
    return bf16_round(rope_rotate(x, base))


def rope_sparse_forward(q, k, v, T, w, scale, base: float = 10000.0, stored: bool = False):
    """sparse_forward on rotated queries and keys (rounded to bf16 as stored when
    `stored`, exact otherwise)."""
    if stored:
        return sparse_forward(rope_store_bf16(q, base), rope_store_bf16(k, base), v, T, w, scale)
    return sparse_forward(rope_rotate(q, base), rope_rotate(k, base), v, T, w, scale)


def rope_sparse_backward(q, k, v, dout, T, w, scale, base: float = 10000.0, stored: bool = False,
                         o=None, lse=None):
    """Gradients of sum(dout * o) of rope_sparse_forward with respect to the unrotated
    q, k and v: the rotated-input gradients carried back through the transposed
    rotation (chain rule through a linear map; the storage rounding, when `stored`,
    passes gradients unchanged, as a separate rotation step's backward would).
    o and lse, when given, are the forward outputs handed to the backward (see
    sparse_backward)."""
    if stored:
        qr, kr = rope_store_bf16(q, base), rope_store_bf16(k, base)
    else:
        qr, kr = rope_rotate(q, base), rope_rotate(k, base)
    dq, dk, dv = sparse_backward(qr, kr, v, dout, T, w, scale, o=o, lse=lse)
    return rope_rotate(dq, base, inverse=True), rope_rotate(dk, base, inverse=True), dv


def _rotate_rows_back(x, rows, N, d, base):
    ang = rope_angles(N, d, base)[np.asarray(rows)]
    c, s = np.cos(ang), -np.sin(ang)
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return out


def rope_sparse_forward_rows(q, k, v, T, w, scale, rows, base: float = 10000.0, stored: bool = False):
    """Rows of rope_sparse_forward."""
    rot = _rope_rot(base, stored)
    return sparse_forward_rows(rot(q), rot(k), v, T, w, scale, rows)


def rope_sparse_backward_rows(q, k, v, dout, T, w, scale, rows, base: float = 10000.0, stored: bool = False):
    """Rows of rope_sparse_backward."""
    N, d = np.asarray(q).shape[-2], np.asarray(q).shape[-1]
    rot = _rope_rot(base, stored)
    dq, dk, dv = sparse_backward_rows(rot(q), rot(k), v, dout, T, w, scale, rows)
    return _rotate_rows_back(dq, rows, N, d, base), _rotate_rows_back(dk, rows, N, d, base), dv


def _rope_rot(base, stored):
    return (lambda x: rope_store_bf16(x, base)) if stored else (lambda x: rope_rotate(x, base))


def rope_frac_forward(q, k, v, entries, w, scale, base: float = 10000.0, stored: bool = False):
    """The learned-alpha variant as the pages run it: queries and keys rotated first
    ([EXPL-pt] Metodologia / Arquitetura, item "Implementação"), then frac_forward, so
    each entry interpolates rotated key rows (values are not rotated)."""
    rot = _rope_rot(base, stored)
    return frac_forward(rot(q), rot(k), v, entries, w, scale)


def rope_frac_backward(q, k, v, dout, entries, w, scale, base: float = 10000.0, stored: bool = False,
                       o=None, lse=None):
    """Gradients of rope_frac_forward: frac_backward on the rotated rows, dq and dk
    rotated back (the transpose), dv and the per-entry derivative unchanged."""
    rot = _rope_rot(base, stored)
    dq, dk, dv, dd = frac_backward(rot(q), rot(k), v, dout, entries, w, scale, o=o, lse=lse)
    return rope_rotate(dq, base, inverse=True), rope_rotate(dk, base, inverse=True), dv, dd
