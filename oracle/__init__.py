"""fp64 CPU oracle for the Dion3 orthogonalization hot path.

Test infrastructure only: imported by tests/, by the smoke check in
__graft_entry__.py and by the CPU-baseline leg of bench.py, never by the
product package.
"""
from .dion_oracle import (  # noqa: F401
    DEFAULT_COEFFS,
    apply_factor,
    coefficient_schedule,
    gram,
    gram_newton_schulz,
    gram_polynomial,
    momentum_update,
    orthogonalize,
    orthogonalize_batch,
    rel_frobenius,
    restart_points,
    row_keys,
    row_keys_fsum,
    round_to_bf16,
    rowsubset_step,
    rowsubset_step_update,
    select_rows,
    selected_count,
    weight_update_f32,
)
