"""fp64 CPU oracle for Fibonacci-offset sparse attention.

Test infrastructure only: imported by tests/, the package smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""
from .fsa_ref import (  # noqa: F401
    attended_offsets,
    coprime_layer,
    dense_forward,
    dense_forward_rows,
    fibonacci_base,
    frac_alpha_grad,
    frac_backward,
    frac_backward_rows,
    frac_forward,
    frac_forward_rows,
    frac_offset_table,
    frac_probabilities,
    offset_table,
    pow2_base,
    rope_angles,
    rope_frac_backward,
    rope_frac_forward,
    rope_rotate,
    rope_sparse_backward,
    rope_sparse_backward_rows,
    rope_sparse_forward,
    rope_sparse_forward_rows,
    rope_store_bf16,
    rope_table_f32,
    round_half_away,
    round_half_even,
    sparse_backward,
    sparse_backward_rows,
    sparse_forward,
    sparse_forward_rows,
    sparse_probabilities,
    stagger_alpha,
)
