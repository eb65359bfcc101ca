"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Holds no attention arithmetic: it draws N(0, 1) values with a CPU generator (or,
for the largest inputs, a generator on the device), rounds them to the requested
dtype and returns the tensors. Seed of tensor t in
layer l of workload c: 1_000_000 * c + 1000 * l + t, with t = 0 (Q), 1 (K),
2 (V), 3 (dO).
"""
from __future__ import annotations

import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3}


def seed_of(workload: int, layer: int, tensor: str) -> int:
    return 1_000_000 * workload + 1000 * layer + TENSOR_IDS[tensor]


def normal(shape, seed: int, dtype=torch.float32) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32).to(dtype)


def normal_on(device, shape, seed: int, dtype=torch.float32) -> torch.Tensor:
    """As normal(), drawn by a generator on `device` (for inputs of several GiB, which a
    CPU generator draws slowly); returns a tensor on that device."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device).to(dtype)


def layer_inputs(workload: int, layer: int, shape, dtype, with_grad: bool = False) -> dict:
    """CPU tensors q, k, v (and do) for one layer of a workload."""
    names = ("q", "k", "v", "do") if with_grad else ("q", "k", "v")
    return {t: normal(shape, seed_of(workload, layer, t), dtype) for t in names}


def as_f64(t: torch.Tensor):
    """Exact float64 numpy copy of a (CPU or device) tensor, for the oracle."""
    return t.detach().to("cpu", torch.float64).numpy()
