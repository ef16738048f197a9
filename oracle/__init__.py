"""CPU oracle for MLA decode attention (test infrastructure only).

Imported by the tests, the smoke check and the bench's CPU-baseline leg, never
by the product path.  It shares no code with the HIP kernels.
"""
from .mla_oracle import (  # noqa: F401
    PAGE, D_QK, D_V, widen, visible_keys, gather_rows, check_lengths, attend_one,
    mla_decode, softmax_weights, weights_and_lse, merge_partials, brute_force, selected_rows,
    mla_decode_sparse, mla_decode_fp8, fp8_rows, fp8_scale_in_format, kv_append,
)
