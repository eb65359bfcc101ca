"""Builds libfsa.so (C-ABI host layer + HIP kernels for gfx950) in-tree with hipcc.

Usage: python -m fibonacci_offset_transformer_amd.build [--verbose]
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfsa.so")

SOURCES = ["fsa_abi.cpp", "fsa_forward.hip", "fsa_backward.hip", "fsa_decode.hip", "fsa_rope.hip", "fsa_noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def command(out: str = LIB) -> list[str]:
    return [
        hipcc(),
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-Wall",
        # packed fp32 VALU ops are kept out of the generated code on purpose
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # no implicit multiply-add fusion: the kernels write every fma they use, so the
        # rounding of each step is the same in every instantiation and call site
        "-ffp-contract=off",
        # MFMA accumulators in ordinary VGPRs: the kernels also update them with VALU
        # ops, and the AGPR form would copy them back and forth around every MFMA
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-I", INCLUDE,
        "-I", CSRC,
        "-o", out,
    ] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False) -> str:
    """Compiles every source into libfsa.so next to this file; returns its path."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in ln]  # the host pass does not know the device feature
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
