"""Fibonacci-offset sparse attention for AMD MI355X (gfx950).

The computation lives in libfsa.so (hand-written HIP kernels behind a C ABI,
declared in include/fsa.h); this package binds it with ctypes.
"""
from .fsa import (  # noqa: F401
    EXPORTS,
    FsaError,
    backward,
    backward_delta,
    backward_grads,
    build_offsets,
    dense_forward,
    forward,
    library,
)
from . import schedules, synth  # noqa: F401
