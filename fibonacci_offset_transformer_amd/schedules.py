"""Per-layer alpha schedules of the pages (host-side configuration).

Page "Depth-Staggered Fibonacci Spacing for Sparse Attention: Static Schedules
Beat Learned Dilation and Extrapolate Where Dense Attention Fails" (gist.science
explainer), section "Variáveis Experimentais": fixed alpha = 1 in every layer;
a static linear ramp from 0.5 at the first layer to 1.5 at the last; and the
same multiset of alphas reassigned by the coprime step layer -> 7 * layer mod L.
Section "Controles": the reach-matched power-of-2 base (table base "pow2").
"""
from __future__ import annotations


def fixed(n_layers: int = 16, alpha: float = 1.0) -> list[float]:
    return [float(alpha)] * n_layers


def linear_stagger(n_layers: int = 16, lo: float = 0.5, hi: float = 1.5) -> list[float]:
    """alpha_l = lo + l * (hi - lo) / (L - 1), evaluated in that order in fp64."""
    if n_layers == 1:
        return [float(lo)]
    return [lo + (l * (hi - lo)) / (n_layers - 1) for l in range(n_layers)]


def literal_stagger(n_layers: int = 16) -> list[float]:
    """The stagger formula as one workload description writes it, alpha_l = 0.5 +
    l * (1.5 / 15) (fp64, in that order). It reaches 2.0 at layer 15, outside the
    pages' alpha range [0.5, 1.5]; it is run once beside the ramp, not instead of it."""
    return [0.5 + l * (1.5 / 15) for l in range(n_layers)]


def coprime_stagger(n_layers: int = 16, step: int = 7, lo: float = 0.5, hi: float = 1.5) -> list[float]:
    """Layer l takes the linear-stagger alpha of layer step * l mod L."""
    lin = linear_stagger(n_layers, lo, hi)
    return [lin[(step * l) % n_layers] for l in range(n_layers)]
