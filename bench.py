#!/usr/bin/env python3
"""Throughput of Fibonacci-offset sparse attention on one MI355X.

Workload: the 16-layer training step at 4x extrapolation: for each of 16 layers,
sparse forward + backward on bf16 Q, K, V, dO of shape [B=2, H=8, N=4096, d=64]
with the static linear stagger alpha_l = 0.5 + l/15 (Fibonacci base, window
w = 64, reach R = 1024; tables built at R = 1024 and used unchanged at 4096).
Inputs are seeded N(0, 1) synthetic tensors resident in HBM before timing.

One step = a training step's attention work: the 16 layers' fsa_forward in layer
order, then their fsa_backward (the whole backward: D, dQ and the pair weights, dK
and dV) in reverse layer order, launched as one HIP graph. Prints one JSON line:
query-heads/s (value), algorithmic HBM GB/s of the step, a roofline entry for the
dominant kernel, the step in per-layer order (forward then backward of each layer)
and after writing 1 GiB of scratch (cold caches), the forward at the training length
N = 1024 (one layer of bf16 [8,8,1024,64], and the 16-layer stagger), the dense
causal baseline, device-copy rates on buffers the last-level cache cannot hold (a
1 GiB copy, and per stage copies moving its bytes per launch) for reference, and the
fp64 CPU oracle timed on a bounded sample of the same workload.

The learned-alpha variant (fractional targets, interpolated K/V rows) and the
rotary-embedding variant (unrotated Q, K in) are timed on the same layers next to
the static path, and so are the pages' other schedules (the coprime reassignment,
the power-of-2 base with the stagger, the window sweep).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--no-dense] [--no-decode] [--no-frac] [--no-rope] [--no-literal] [--no-long]
                       [--no-schedules] [--no-cold] [--no-short] [--copy-probe]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn fwd+bwd query-heads/s and achieved HBM GB/s at N=1024/4096, 1 GPU"
B, H, N, D, LAYERS, W, R, BASE = 2, 8, 4096, 64, 16, 64, 1024, "fib"
WORKLOAD_ID = 4
HBM_PEAK_GBS = 8000.0
# worker processes of the CPU baseline: the host's CPU share per GPU on the measurement
# boxes (16 cores for one GPU), whatever the process can see
HOST_CPU_SHARE = 16
BF16_MFMA_PEAK_TFLOPS = 2500.0
ELEM = 2  # bf16 bytes


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- algorithmic figures

def rows_per_layer():
    return B * H * N


def alg_bytes_per_row():
    """Compulsory HBM bytes per (b, h, row) of each stage and of the whole step.

    fwd:  read q, k, v; write o, lse
    bwd:  read q, k, v, o, dO, lse; write dq, dk, dv (the D and pair-weight
          workspaces are the library's scratch and not counted)
    step (fwd + bwd, each tensor element once):
          read q, k, v, o, dO, lse; write o, lse, dq, dk, dv
    """
    row = D * ELEM
    return {
        "fwd": 4 * row + 4,
        "bwd": 8 * row + 4,
        "step": 12 * row + 8,
    }


def band_keys_per_head():
    """Sum over rows of the window keys a row attends, min(i + 1, w)."""
    return sum(min(i + 1, W) for i in range(N))


def band_flops_per_layer():
    """Useful window-band flops per layer: forward 2 products (scores, P.V), backward 5
    (scores, dP, dV, dQ, dK), 2 d flops each per (query, key) pair."""
    pairs = B * H * band_keys_per_head()
    return {"fwd": 4 * D * pairs, "bwd": 10 * D * pairs}


def dense_flops_per_layer():
    # causal: 2 products of 2*d flops for each of the N(N+1)/2 (query, key) pairs, per head
    return B * H * 4 * D * (N * (N + 1) // 2)


# ---------------------------------------------------------------- CPU baseline (oracle)

_SAMPLE = []  # (q, k, v, dO, table) per sampled head; filled before the worker pool forks


def _oracle_head(idx):
    import oracle
    q, k, v, do, T = _SAMPLE[idx]
    oracle.sparse_forward(q, k, v, T, W, 1.0 / math.sqrt(D))
    oracle.sparse_backward(q, k, v, do, T, W, 1.0 / math.sqrt(D))
    return q.shape[0]


def cpu_baseline(cpu_inputs, alphas, heads_per_core=8):
    """fp64 numpy oracle (sparse forward + backward) on sampled heads, one process per core."""
    import multiprocessing as mp

    import numpy as np
    import torch

    import oracle

    visible = len(os.sched_getaffinity(0))
    cores = max(1, min(HOST_CPU_SHARE, visible))
    n_heads = cores * heads_per_core
    rng = np.random.default_rng(7)
    _SAMPLE.clear()
    for t in range(n_heads):
        l = t % LAYERS
        b, h = int(rng.integers(0, B)), int(rng.integers(0, H))
        x = cpu_inputs[l]
        T = oracle.offset_table(BASE, alphas[l], W, R)
        _SAMPLE.append(tuple(x[n][b, h].to(torch.float64).numpy() for n in ("q", "k", "v", "do")) + (T,))
    os.environ["OMP_NUM_THREADS"] = "1"
    ctx = mp.get_context("fork")
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_head, range(cores), chunksize=1)  # warm the workers (imports, caches)
        t0 = time.perf_counter()
        rows = sum(pool.map(_oracle_head, range(n_heads), chunksize=1))
        wall = time.perf_counter() - t0
    _SAMPLE.clear()
    try:
        model = next(ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name"))
    except Exception:
        model = "unknown"
    return {
        "value": rows / wall,
        "unit": "query-heads/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{n_heads} of {LAYERS * B * H} (layer, b, h) heads of the same workload, fp64 numpy "
                  f"sparse forward + backward at N={N}, {cores} single-threaded worker processes "
                  f"(the host's CPU share per GPU; {visible} cores visible to the process), "
                  f"{wall:.2f} s wall ({wall * cores:.1f} core-seconds); CPU: {model}",
        "cores_visible": visible,
    }


# ---------------------------------------------------------------- GPU part

# The sources the kernels are compiled from, in a fixed order.
KERNEL_SOURCES = ("fsa_internal.h", "fsa_device.h", "fsa_forward.hip", "fsa_backward.hip", "fsa_decode.hip",
                  "fsa_rope.hip")


def kernel_source_sha():
    """Hash of the kernel sources' code, comments and blank lines left out (the sources
    hold no string literal with a comment marker), so that a comment edit keeps the
    counter readings taken on the same code."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        text = open(os.path.join(ROOT, "fibonacci_offset_transformer_amd", "csrc", name)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = (re.sub(r"//.*", "", line).rstrip() for line in text.split("\n"))
        h.update("\n".join(line for line in lines if line).encode())
    return h.hexdigest()


# Kernels that one launch of each stage runs (bf16, window path, B * H a multiple of 8:
# the backward's dQ and dK/dV work in one launch), under their short names.
STAGE_KERNELS = {"fwd": ("fwd",), "bwd": ("bwd",)}
KERNEL_NAMES = {"fwd": "fwd_window_kernel<bf16 out>", "bwd": "bwd_fused_kernel<bf16 out, D formed>"}


def measured_traffic(stage):
    """HBM bytes per launch of a stage (summed over its kernels) from committed rocprofv3
    counter readings, if they were taken on the current kernel source; None otherwise."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(p))
    except Exception:
        return None
    if rec.get("kernel_source_sha256") != kernel_source_sha():
        return None
    total = 0.0
    for name in STAGE_KERNELS[stage]:
        k = rec.get("kernels", {}).get(name)
        if not k:
            return None
        total += k["fetch_kib_per_dispatch"] * 1024.0 * rec["copy_scale_fetch"]
        total += k["write_kib_per_dispatch"] * 1024.0 * rec["copy_scale_write"]
    return total


# decode: the newest token of each of DEC_B sequences against full caches of DEC_LMAX rows
DEC_B, DEC_LMAX, DEC_ALPHA = 64, 4096, 1.0
DEC_FRAC_ALPHA = 1.0 + 1.0 / 15  # a learned value near the learned variant's start (alpha = 1): unrounded targets


def decode_keys(table, w, L):
    """Keys one decode query attends: the window's min(w, L) plus table entries <= L - 1."""
    return min(w, L) + sum(1 for o in table if o <= L - 1)


def decode_bench(fsa, torch, dev, stream):
    """Sparse decode (window 64 + Fibonacci offsets), dense decode (window = cache) and the
    learned-alpha variant's decode (fractional targets, two cached rows per entry) at the
    same shapes: microseconds per step and algorithmic bytes per second."""
    from fibonacci_offset_transformer_amd import synth
    x = synth.layer_inputs(6, 0, (DEC_B, H, DEC_LMAX, D), torch.bfloat16, with_grad=True)
    k, v = x["k"].to(dev), x["v"].to(dev)
    q = x["q"][:, :, -1].contiguous().to(dev)
    del x
    sl = torch.full((DEC_B,), DEC_LMAX, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((DEC_B, H), dtype=torch.float32, device=dev)
    res = {"config": {"sequences": DEC_B, "heads": H, "cache_rows": DEC_LMAX, "head_dim": D, "dtype": "bf16",
                      "base": BASE, "alpha": DEC_ALPHA, "R": R}}
    for name, w, alpha, frac in (("sparse", W, DEC_ALPHA, False), ("dense", DEC_LMAX, DEC_ALPHA, False),
                                 ("learned_alpha", W, DEC_FRAC_ALPHA, True)):
        if frac:  # each entry reads two cached rows
            ents = [(a, ph) for a, ph, _ in fsa.frac_offsets(alpha, w, R, BASE)]
            n_ent = sum(1 for a, ph in ents if a + (ph != 0.0) <= DEC_LMAX - 1)
            keys = min(w, DEC_LMAX) + n_ent
            rows_read = min(w, DEC_LMAX) + 2 * n_ent
        else:
            table = fsa.build_offsets(alpha, w, R, BASE)
            keys = decode_keys(table, w, DEC_LMAX)
            rows_read = keys
        step_bytes = DEC_B * H * (rows_read * 2 * D * ELEM + 2 * D * ELEM + 4)

        def run():
            fsa.decode(q, k, v, sl, alpha=alpha, w=w, R=R, base=BASE, out=o, lse=lse, fractional=frac)

        run()
        torch.cuda.synchronize()
        reps = 50
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        eager_us = e0.elapsed_time(e1) * 1e3 / reps
        # device time: the steps captured back to back in a HIP graph (no host launch gaps)
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            run()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                run()
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        del g
        res[name] = {"window": w, "alpha": alpha, "keys_per_query": keys, "us_per_step": round(us, 2),
                     "us_per_step_eager": round(eager_us, 2),
                     "algorithmic_bytes": step_bytes, "gb_s": round(step_bytes / (us * 1e-6) / 1e9, 1)}
    res["dense_over_sparse_time"] = round(res["dense"]["us_per_step"] / res["sparse"]["us_per_step"], 2)
    res["learned_alpha_over_sparse_time"] = round(res["learned_alpha"]["us_per_step"] / res["sparse"]["us_per_step"], 3)
    return res


def long_context_bench(fsa, torch, dev, stream, scale, reps):
    """One layer of the power-of-2 control at 8x the sequence length: bf16 [1, 8, 32768, 64],
    table [64, 128, 256, 512] (w = 64, R = 1024), forward and backward, each timed as a HIP
    graph of 10 launches."""
    from fibonacci_offset_transformer_amd import synth
    Bl, Hl, Nl = 1, 8, 32768
    x = {k: t.to(dev) for k, t in synth.layer_inputs(5, 0, (Bl, Hl, Nl, D), torch.bfloat16, with_grad=True).items()}
    kw = dict(alpha=1.0, w=W, R=R, base="pow2", scale=scale)
    o = torch.empty_like(x["q"])
    lse = torch.empty((Bl, Hl, Nl), dtype=torch.float32, device=dev)
    dl = torch.empty_like(lse)
    g = [torch.empty_like(x["q"]) for _ in range(3)]
    pw = torch.empty(max(fsa.workspace_bytes(torch.bfloat16, Bl, Hl, Nl, D, **{k: kw[k] for k in ("alpha", "w", "R",
                                                                                                   "base")}), 16) // 4,
                     dtype=torch.int32, device=dev)

    def fwd():
        fsa.forward(x["q"], x["k"], x["v"], out=o, lse=lse, **kw)

    def bwd():
        fsa.backward(x["q"], x["k"], x["v"], o, lse, x["do"], dq=g[0], dk=g[1], dv=g[2], delta=dl, pair_ws=pw, **kw)

    res = {}
    for name, fn in (("fwd", fwd), ("bwd", bwd)):
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            fn()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for _ in range(10):
                fn()
        for _ in range(3):
            gr.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            gr.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1e3 / (reps * 10)
    rows = Bl * Hl * Nl
    per_row = alg_bytes_per_row()
    return {
        "what": "power-of-2 control at 8x the length: bf16 [1,8,32768,64], table [64,128,256,512], one layer",
        "fwd_us": round(res["fwd"], 2), "bwd_us": round(res["bwd"], 2),
        "query_heads_per_s": round(rows / ((res["fwd"] + res["bwd"]) * 1e-6), 1),
        "fwd_gb_s": round(per_row["fwd"] * rows / (res["fwd"] * 1e-6) / 1e9, 1),
        "bwd_gb_s": round(per_row["bwd"] * rows / (res["bwd"] * 1e-6) / 1e9, 1),
    }


def short_context_bench(fsa, torch, dev, stream, reps):
    """The forward at the training length N = 1024 (bf16 [8,8,1024,64], w = 64, R = 1024):
    the one-layer workload (alpha = 1) and the 16-layer linear stagger, each timed as the
    average launch over 16 layers' own seeded inputs (541 MB, more than the 256 MB
    last-level cache, so every launch reads its inputs from HBM); and the fp32
    single-head workload (fp32 [1,1,256,64], w = 16, R = 256): four workgroups, whose
    time is the latency of one workgroup's chain of dependent loads, not bandwidth."""
    from fibonacci_offset_transformer_amd import schedules, synth
    Bs, Hs, Ns = 8, 8, 1024
    shape = (Bs, Hs, Ns, D)
    bufs = []
    for l in range(LAYERS):
        x = {k: t.to(dev) for k, t in synth.layer_inputs(3, l, shape, torch.bfloat16, with_grad=False).items()}
        x["o"] = torch.empty_like(x["q"])
        x["lse"] = torch.empty(shape[:3], dtype=torch.float32, device=dev)
        bufs.append(x)
    alphas = schedules.linear_stagger(LAYERS)
    scale = 1.0 / math.sqrt(D)

    def fwd(alpha_of):
        def run(l):
            x = bufs[l]
            fsa.forward(x["q"], x["k"], x["v"], alpha=alpha_of(l), w=W, R=R, base=BASE, scale=scale, out=x["o"],
                        lse=x["lse"])
        return run

    us_one = stage_us(torch, dev, stream, fwd(lambda l: 1.0), reps)
    us_stagger = stage_us(torch, dev, stream, fwd(lambda l: alphas[l]), reps)
    rows = Bs * Hs * Ns
    nbytes = alg_bytes_per_row()["fwd"] * rows

    def line(us, layers):
        achieved = nbytes / (us * 1e-6) / 1e9
        return {
            "us_per_layer": round(us, 3),
            "us_per_pass": round(us * layers, 3),
            "query_heads_per_s": round(rows / (us * 1e-6), 1),
            "gb_s": round(achieved, 1),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "kernel": KERNEL_NAMES["fwd"],
                         "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": round(us, 3)},
        }

    del bufs
    # fp32 single head: 100 launches captured in one graph
    x1 = {k: t.to(dev) for k, t in synth.layer_inputs(1, 0, (1, 1, 256, D), torch.float32, with_grad=False).items()}
    o1 = torch.empty_like(x1["q"])
    l1 = torch.empty((1, 1, 256), dtype=torch.float32, device=dev)

    def one():
        fsa.forward(x1["q"], x1["k"], x1["v"], alpha=1.0, w=16, R=256, base=BASE, scale=scale, out=o1, lse=l1)

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        one()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(100):
            one()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us1 = e0.elapsed_time(e1) * 1e3 / 500
    del g
    return {
        "what": "forward at the training length N = 1024: bf16 [8,8,1024,64], w = 64, R = 1024; each figure the "
                "average launch over 16 layers' own seeded inputs (read from HBM)",
        "one_layer_alpha1": line(us_one, 1),
        "sixteen_layer_stagger": line(us_stagger, LAYERS),
        "fp32_single_head": {"what": "fp32 [1,1,256,64], w = 16, alpha = 1, R = 256, forward (general kernel; "
                                     "latency-bound: 4 workgroups)",
                             "us_per_launch": round(us1, 3),
                             "query_heads_per_s": round(256 / (us1 * 1e-6), 1)},
    }


def copy_reference(torch, dev, stream, stage_bytes):
    """Device-copy rates (bytes read + written per second) for reference, always on buffers
    that the 256 MB last-level cache cannot hold from one pass to the next: a 1 GiB to
    1 GiB copy (the sustained rate), and for each stage copies that move its algorithmic
    bytes per launch (half read, half written), rotated over 16 distinct buffer pairs
    like the layers of the step."""
    def rate(pairs, reps):
        for s, d in pairs:
            d.copy_(s)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            for s, d in pairs:
                d.copy_(s)
        e1.record(stream)
        torch.cuda.synchronize()
        moved = 2 * reps * sum(s.numel() * s.element_size() for s, _ in pairs)
        return moved / (e0.elapsed_time(e1) * 1e-3) / 1e9

    src = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    out = {"large_gb_s": round(rate([(src, dst)], 5), 1)}
    del src, dst
    for k, nbytes in stage_bytes.items():
        elems = int(nbytes) // 2 // 4
        pairs = [(torch.ones(elems, dtype=torch.float32, device=dev), torch.empty(elems, dtype=torch.float32, device=dev))
                 for _ in range(LAYERS)]
        out[f"{k}_sized_gb_s"] = round(rate(pairs, 5), 1)
        del pairs
    out["what"] = ("torch device-to-device copies (the HIP runtime's copy kernel); large: 1 GiB to 1 GiB; "
                   "<stage>_sized: 16 distinct buffer pairs, each copy moving that stage's algorithmic bytes per launch "
                   "(at the forward's 34 MB a copy launch does not reach the sustained rate)")
    return out


def stage_us(torch, dev, stream, fn, reps):
    """Average duration (us) of one layer's launches of fn: the 16 layers captured back to
    back in a HIP graph, replayed `reps` times (after ten untimed replays) between two
    HIP events on the stream."""
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for l in range(LAYERS):
            fn(l)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for l in range(LAYERS):
            fn(l)
    # a freshly instantiated graph runs its first replays slower: leave ten untimed
    for _ in range(10):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * LAYERS)


def frac_bench(fsa, torch, dev, stream, bufs, alphas, scale, static_us, reps):
    """The learned-alpha variant on the same 16 layers: the stagger alphas taken as learned
    values, so every target alpha*F stays unrounded and each entry reads interpolated
    K/V rows. Per-layer forward and backward (dQ, dK/dV, alpha gradient) durations next
    to the static path's."""
    ws_bytes = max(fsa.frac_workspace_bytes(torch.bfloat16, B, H, N, D, alpha=a, w=W, R=R, base=BASE)
                   for a in alphas)
    ws = torch.empty(ws_bytes // 4 + 1, dtype=torch.int32, device=dev)
    dalpha = torch.empty((LAYERS, 1), dtype=torch.float32, device=dev)
    doffs = torch.empty((LAYERS, 48), dtype=torch.float32, device=dev)

    def fwd(l):
        x = bufs[l]
        fsa.frac_forward(x["q"], x["k"], x["v"], alpha=alphas[l], w=W, R=R, base=BASE, scale=scale,
                         out=x["o"], lse=x["lse"])

    def bwd(l):
        x = bufs[l]
        fsa.frac_backward(x["q"], x["k"], x["v"], x["o"], x["lse"], x["do"], alpha=alphas[l], w=W, R=R,
                          base=BASE, scale=scale, dq=x["dq"], dk=x["dk"], dv=x["dv"], dalpha=dalpha[l],
                          doffs=doffs[l], ws=ws)

    def step(l):
        fwd(l)
        bwd(l)

    fwd_us = stage_us(torch, dev, stream, fwd, reps)
    bwd_us = stage_us(torch, dev, stream, bwd, reps)
    step_us = stage_us(torch, dev, stream, step, reps)
    entries = [len(fsa.frac_offsets(a, W, R, BASE)) for a in alphas]
    return {
        "what": "learned-alpha variant: fractional targets alpha*F (stagger alphas taken unrounded), "
                "keys/values interpolated between the two rows around each target, fused in the "
                "window kernels; dK/dV/dQ plus d(loss)/d(alpha)",
        "entries_per_layer": entries,
        "fwd_us_per_layer": round(fwd_us, 3),
        "bwd_us_per_layer": round(bwd_us, 3),
        "static_fwd_us_per_layer": round(static_us["fwd"], 3),
        "static_bwd_us_per_layer": round(static_us["bwd"], 3),
        "fwd_over_static": round(fwd_us / static_us["fwd"], 3),
        "bwd_over_static": round(bwd_us / static_us["bwd"], 3),
        "step_us_per_layer": round(step_us, 3),
        "static_step_us_per_layer": round(static_us["step"], 3),
        "step_over_static": round(step_us / static_us["step"], 3),
    }


def rope_bench(fsa, torch, dev, stream, bufs, alphas, scale, static_us, reps):
    """Rotary embedding before the attention on the same 16 layers (unrotated Q, K in,
    gradients with respect to them out): per-layer forward and backward durations
    next to the static path's, and the rotation pass alone."""
    table = fsa.rope_table(N, D, device=dev)
    f_bytes, b_bytes = zip(*(fsa.rope_workspace_bytes(torch.bfloat16, B, H, N, D, alpha=a, w=W, R=R, base=BASE)
                             for a in alphas))
    ws = torch.empty(max(b_bytes) // 4 + 1, dtype=torch.int32, device=dev)

    def fwd(l, keep=False):  # inference: the rotated Q is not kept
        x = bufs[l]
        fsa.rope_forward(x["q"], x["k"], x["v"], table, alpha=alphas[l], w=W, R=R, base=BASE, scale=scale,
                         out=x["o"], lse=x["lse"], ws=ws, keep_rotated=keep)

    def bwd(l):
        x = bufs[l]
        fsa.rope_backward(x["q"], x["k"], x["v"], table, x["o"], x["lse"], x["do"], alpha=alphas[l], w=W, R=R,
                          base=BASE, scale=scale, dq=x["dq"], dk=x["dk"], dv=x["dv"], ws=ws)

    def step(l):  # a training step keeps the forward's rotated rows for its backward
        fwd(l, keep=True)
        x = bufs[l]
        fsa.rope_backward(x["q"], x["k"], x["v"], table, x["o"], x["lse"], x["do"], alpha=alphas[l], w=W, R=R,
                          base=BASE, scale=scale, dq=x["dq"], dk=x["dk"], dv=x["dv"], ws=ws, reuse_rotated=True)

    def rot(l):
        x = bufs[l]
        fsa.rope_rotate(x["q"], table, out=x["dq"])

    fwd_us = stage_us(torch, dev, stream, fwd, reps)
    bwd_us = stage_us(torch, dev, stream, bwd, reps)
    step_us = stage_us(torch, dev, stream, step, reps)
    rot_us = stage_us(torch, dev, stream, rot, reps)
    rot_bytes = B * H * N * (2 * D * ELEM)  # one tensor: read and write each row (the table stays in L2)
    return {
        "what": "rotary embedding before the attention: the forward kernel rotates its query rows and its "
                "tiles' K rows (bf16, as a separate rotation step stores them; each tile stores its own rotated "
                "K rows for the other tiles' slabs and for the backward), the backward reuses the forward's "
                "rotated rows or rotates them in a pass, and rotates dQ and dK back in its store",
        "fwd_us_per_layer": round(fwd_us, 3),
        "bwd_us_per_layer": round(bwd_us, 3),
        "static_fwd_us_per_layer": round(static_us["fwd"], 3),
        "static_bwd_us_per_layer": round(static_us["bwd"], 3),
        "fwd_over_static": round(fwd_us / static_us["fwd"], 3),
        "bwd_over_static": round(bwd_us / static_us["bwd"], 3),
        "step_us_per_layer": round(step_us, 3),
        "step_note": "forward, then the backward reusing the forward's rotated rows",
        "static_step_us_per_layer": round(static_us["step"], 3),
        "step_over_static": round(step_us / static_us["step"], 3),
        "rotation_us_per_tensor": round(rot_us, 3),
        "rotation_gb_s": round(rot_bytes / (rot_us * 1e-6) / 1e9, 1),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-frac", action="store_true", help="skip the learned-alpha (fractional) variant")
    ap.add_argument("--no-rope", action="store_true", help="skip the rotary-embedding variant")
    ap.add_argument("--no-long", action="store_true", help="skip the [1,8,32768,64] power-of-2 layer")
    ap.add_argument("--no-literal", action="store_true",
                    help="skip the run with the literal stagger formula 0.5 + l*(1.5/15)")
    ap.add_argument("--no-schedules", action="store_true",
                    help="skip the steps under the coprime, power-of-2 stagger and window-sweep schedules")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the single steps timed after writing 1 GiB of scratch (cold caches)")
    ap.add_argument("--no-short", action="store_true",
                    help="skip the forward at the training length N = 1024 (bf16 [8,8,1024,64], one layer and "
                         "the 16-layer stagger) and the fp32 single-head case")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter scale reference) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "this library runs the sparse-attention path on one GPU and does not shard it.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 3}))
        return

    from fibonacci_offset_transformer_amd import fsa, schedules, synth

    alphas = schedules.linear_stagger(LAYERS)
    log(f"generating inputs: {LAYERS} layers x bf16 [{B},{H},{N},{D}] (q, k, v, dO)")
    cpu_inputs = [synth.layer_inputs(WORKLOAD_ID, l, (B, H, N, D), torch.bfloat16, with_grad=True)
                  for l in range(LAYERS)]

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample (before any GPU use)")
        cpu = cpu_baseline(cpu_inputs, alphas)
        log(f"cpu baseline: {cpu['value']:.1f} query-heads/s on {cpu['cores']} cores")

    dev = torch.device("cuda:0")
    bufs = []
    for l in range(LAYERS):
        x = {k: t.to(dev) for k, t in cpu_inputs[l].items()}
        x["o"] = torch.empty_like(x["q"])
        x["lse"] = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        x["delta"] = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        for g in ("dq", "dk", "dv"):
            x[g] = torch.empty_like(x["q"])
        bufs.append(x)
    del cpu_inputs
    scale = 1.0 / math.sqrt(D)
    tables = [fsa.build_offsets(a, W, R, BASE) for a in alphas]
    # one pair workspace serves every layer (the layers run one after another on the stream)
    pair_bytes = max(fsa.workspace_bytes(torch.bfloat16, B, H, N, D, alpha=a, w=W, R=R, base=BASE) for a in alphas)
    pair_ws = torch.empty(max(pair_bytes, 16) // 4, dtype=torch.int32, device=dev)
    log("offset tables per layer: " + "; ".join(",".join(map(str, t)) for t in tables))

    def layer_fwd(l):
        x = bufs[l]
        fsa.forward(x["q"], x["k"], x["v"], alpha=alphas[l], w=W, R=R, base=BASE, scale=scale,
                    out=x["o"], lse=x["lse"])

    def layer_bwd(l):
        x = bufs[l]
        fsa.backward(x["q"], x["k"], x["v"], x["o"], x["lse"], x["do"], alpha=alphas[l], w=W, R=R, base=BASE,
                     scale=scale, dq=x["dq"], dk=x["dk"], dv=x["dv"], delta=x["delta"], pair_ws=pair_ws)

    def step():
        # a training step: every layer's forward in layer order, then the backward from
        # the last layer down, so each backward finds its layer's rows long evicted
        for l in range(LAYERS):
            layer_fwd(l)
        for l in reversed(range(LAYERS)):
            layer_bwd(l)

    def step_per_layer():
        # forward then backward of each layer in turn (each backward finds its layer's
        # rows still in the last-level cache): reported beside the training step
        for l in range(LAYERS):
            layer_fwd(l)
            layer_bwd(l)

    # eager reference results
    step()
    torch.cuda.synchronize()
    ref = [tuple(bufs[l][t].clone() for t in ("o", "lse", "dq", "dk", "dv")) for l in range(LAYERS)]

    stream = torch.cuda.current_stream(dev)

    def capture(fn):
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            fn()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    # one step captured as a HIP graph
    graph = capture(step)
    graph_per_layer = capture(step_per_layer)

    # bring the GPU to steady clocks before anything is timed (untimed replays for at
    # least half a second), then the requested warmup steps
    t_spin = time.perf_counter()
    while time.perf_counter() - t_spin < 0.5:
        for _ in range(20):
            graph.replay()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()

    def timed(g, n):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(n):
            g.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n

    ms_per_step = timed(graph, args.steps)

    # graph replays must reproduce the eager results bit for bit (deterministic kernels)
    for l in range(LAYERS):
        for name, a in zip(("o", "lse", "dq", "dk", "dv"), ref[l]):
            if not torch.equal(bufs[l][name], a):
                raise SystemExit(f"graph replay differs from eager result: layer {l} {name}")

    # per-stage durations (at steady clocks, after the timed steps): each stage's 16
    # per-layer launches captured back to back in a HIP graph of their own, replayed
    # between two HIP events on the launch stream
    reps = max(20, args.steps // 5)
    avg_us = {key: stage_us(torch, dev, stream, fn, reps)
              for key, fn in (("fwd", layer_fwd), ("bwd", layer_bwd))}
    log("average kernel durations (us): " + ", ".join(f"{k}={v:.2f}" for k, v in avg_us.items()))

    def layer_step(l):
        layer_fwd(l)
        layer_bwd(l)

    # forward + backward of one layer back to back (which finds the layer's rows still
    # in cache): the reference for the variants' steps
    static_step_us = stage_us(torch, dev, stream, layer_step, reps)

    # the whole step in per-layer order, for comparison with the training order
    for _ in range(3):
        graph_per_layer.replay()
    per_layer_ms = timed(graph_per_layer, max(5, args.steps // 2))
    del graph_per_layer
    for l in range(LAYERS):
        for name, a in zip(("o", "lse", "dq", "dk", "dv"), ref[l]):
            if not torch.equal(bufs[l][name], a):
                raise SystemExit(f"per-layer order differs from the training-order result: layer {l} {name}")

    # eager step time for context
    step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(max(3, args.steps // 5)):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / max(3, args.steps // 5)

    cold = None
    if not args.no_cold:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        times = []
        for _ in range(max(5, min(args.steps, 20))):
            scratch.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        del scratch
        times.sort()
        cold = {"ms_per_step_median": round(times[len(times) // 2], 5), "steps": len(times),
                "what": "one graph step after writing 1 GiB of scratch, per step"}

    copy_ref = copy_reference(torch, dev, stream, {k: alg_bytes_per_row()[k] * rows_per_layer() for k in avg_us})
    copy_gbs = copy_ref["large_gb_s"]

    def schedule_step(sched_alphas, base, w, reps):
        """ms per training-order step (16 forwards, then 16 backwards in reverse) of the
        same layers' inputs under another schedule, captured as one HIP graph."""
        nbytes = max(fsa.workspace_bytes(torch.bfloat16, B, H, N, D, alpha=a, w=w, R=R, base=base)
                     for a in sched_alphas)
        ws = torch.empty(max(nbytes, 16) // 4, dtype=torch.int32, device=dev)

        def run():
            for l in range(LAYERS):
                x = bufs[l]
                fsa.forward(x["q"], x["k"], x["v"], alpha=sched_alphas[l], w=w, R=R, base=base, scale=scale,
                            out=x["o"], lse=x["lse"])
            for l in reversed(range(LAYERS)):
                x = bufs[l]
                fsa.backward(x["q"], x["k"], x["v"], x["o"], x["lse"], x["do"], alpha=sched_alphas[l], w=w, R=R,
                             base=base, scale=scale, dq=x["dq"], dk=x["dk"], dv=x["dv"], delta=x["delta"],
                             pair_ws=ws)

        g = capture(run)
        for _ in range(3):
            g.replay()
        ms = timed(g, reps)
        del g, ws
        tabs = [fsa.build_offsets(a, w, R, base) for a in sched_alphas]
        return {"ms_per_step": round(ms, 5), "query_heads_per_s": round(rows_per_layer() * LAYERS / (ms * 1e-3), 1),
                "tables_per_layer": [len(t) for t in tabs], "max_offset": max(max(t or [0]) for t in tabs)}

    literal = None
    if not args.no_literal:
        literal = dict(what="the same 16-layer step with alpha_l = 0.5 + l*(1.5/15) as one workload description "
                            "writes it (reaches 2.0 at layer 15; the main run uses the pages' ramp 0.5 + l/15)",
                       **schedule_step(schedules.literal_stagger(LAYERS), BASE, W, max(3, args.steps // 5)))

    other_schedules = None
    if not args.no_schedules:
        reps = max(3, args.steps // 5)
        other_schedules = {
            "what": "the training-order step of the same inputs under the pages' other schedules: the stagger "
                    "reassigned layer -> 7 layer mod 16 (coprime), the power-of-2 base with the linear stagger, and "
                    "the window sweep w = 6, 8, 10, 12 with the Fibonacci stagger (R = 1024 throughout)",
            "coprime": schedule_step(schedules.coprime_stagger(LAYERS), BASE, W, reps),
            "pow2_stagger": schedule_step(alphas, "pow2", W, reps),
        }
        for w_s in (6, 8, 10, 12):
            other_schedules[f"window_{w_s}"] = schedule_step(alphas, BASE, w_s, reps)

    per_row = alg_bytes_per_row()
    rows = rows_per_layer()
    qh_per_step = rows * LAYERS
    step_bytes = per_row["step"] * rows * LAYERS
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    # dominant stage: the backward's two kernels (one launch of fsa_backward runs both)
    dom = max(avg_us, key=lambda k: avg_us[k])
    achieved = per_row[dom] * rows / (avg_us[dom] * 1e-6) / 1e9
    roof = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(dom),
        "kernel": " + ".join(KERNEL_NAMES[k] for k in STAGE_KERNELS[dom]),
        "stage": dom,
        "algorithmic_bytes_per_launch": per_row[dom] * rows,
        "avg_launch_us": round(avg_us[dom], 3),
    }
    band = band_flops_per_layer()
    band_mfma = {k: {"useful_gflop_per_layer": round(band[k] / 1e9, 4),
                     "tflops": round(band[k] / (avg_us[k] * 1e-6) / 1e12, 1),
                     "frac_of_bf16_peak": round(band[k] / (avg_us[k] * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)}
                 for k in ("fwd", "bwd")}
    band_mfma["note"] = ("useful window-band flops (2 products forward, 5 backward, 2 d flops per pair) over the "
                         "stage time; the kernels issue 80 keys per 16-row block (about 1.25x the forward's "
                         "useful flops, and the backward recomputes scores and dP in both kernels)")
    stages = {k: {"avg_us": round(v, 3), "algorithmic_bytes": per_row[k] * rows,
                  "gb_s": round(per_row[k] * rows / (v * 1e-6) / 1e9, 1),
                  "frac_of_runtime_copy_same_bytes": round(per_row[k] * rows / (v * 1e-6) / 1e9
                                                   / copy_ref[f"{k}_sized_gb_s"], 4),
                  "kernels": [KERNEL_NAMES[n] for n in STAGE_KERNELS[k]]} for k, v in avg_us.items()}

    dense = None
    if not args.no_dense:
        od = torch.empty_like(bufs[0]["q"])
        ld = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        for l in range(2):
            fsa.dense_forward(bufs[l]["q"], bufs[l]["k"], bufs[l]["v"], scale=scale, out=od, lse=ld)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        e0.record(stream)
        for _ in range(reps):
            for l in range(LAYERS):
                fsa.dense_forward(bufs[l]["q"], bufs[l]["k"], bufs[l]["v"], scale=scale, out=od, lse=ld)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * LAYERS)
        tflops = dense_flops_per_layer() / (us * 1e-6) / 1e12
        sparse_fwd_us = avg_us["fwd"]
        dense = {
            "what": "dense causal forward, same shapes, one layer",
            "us_per_layer": round(us, 2),
            "tflops": round(tflops, 1),
            "mfma_frac_of_bf16_peak": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "sparse_fwd_us_per_layer": round(sparse_fwd_us, 2),
            "dense_over_sparse_fwd_time": round(us / sparse_fwd_us, 2),
        }

    decode = None
    if not args.no_decode:
        decode = decode_bench(fsa, torch, dev, stream)

    learned = None
    if not args.no_frac:
        learned = frac_bench(fsa, torch, dev, stream, bufs, alphas, scale, dict(avg_us, step=static_step_us),
                             max(3, args.steps // 5))

    long_ctx = None
    if not args.no_long:
        long_ctx = long_context_bench(fsa, torch, dev, stream, scale, 10)

    short = None
    if not args.no_short:
        short = short_context_bench(fsa, torch, dev, stream, max(20, args.steps // 5))

    rope = None
    if not args.no_rope:
        rope = rope_bench(fsa, torch, dev, stream, bufs, alphas, scale, dict(avg_us, step=static_step_us),
                          max(3, args.steps // 5))

    out = {
        "metric": METRIC,
        "value": round(qh_per_step / (ms_per_step * 1e-3), 1),
        "unit": "query-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "16-layer training step at 4x extrapolation: sparse fwd+bwd per layer, bf16 "
                        f"[B={B},H={H},N={N},d={D}], linear stagger alpha_l=0.5+l/15, fib base, w={W}, "
                        f"R={R} (tables reused at N={N}), Q/K/V/dO ~ N(0,1) seeded",
            "layers": LAYERS, "batch": B, "heads": H, "seq_len": N, "head_dim": D,
            "launch": "one HIP graph per step: 16 forwards in layer order, then 16 backwards in reverse "
                      "layer order (2 kernels per layer: the forward and the one-launch backward)",
        },
        "per_layer_order_ms_per_step": round(per_layer_ms, 5),
        "per_layer_order_note": "the same kernels with each layer's backward right after its forward "
                                "(its rows still cached); value and ms_per_step use the training order",
        "hbm_gb_s": round(gbs, 1),
        "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "copy_gb_s": round(copy_gbs, 1),
        "hbm_frac_of_copy": round(gbs / copy_gbs, 4),
        "copy_reference": copy_ref,
        "algorithmic_bytes_per_step": step_bytes,
        "query_heads_per_step": qh_per_step,
        "eager_ms_per_step": round(eager_ms, 4),
        "stages": stages,
        "band_mfma": band_mfma,
        "roofline": roof,
        "cpu_baseline": cpu,
        "dense_baseline": dense,
        "decode": decode,
        "learned_alpha": learned,
        "rope": rope,
        "literal_stagger": literal,
        "schedules": other_schedules,
        "short_context": short,
        "long_context": long_ctx,
        "cold": cold,
    }
    if cpu:
        out["gpu_over_cpu"] = round(out["value"] / cpu["value"], 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
