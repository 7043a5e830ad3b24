"""fp64 CPU oracle for causal ALiBi attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path (the HIP library and its Python binding) never
imports, calls or links anything here, and this package never imports the
product path: the two share no code. Inputs for both come from the seeded
generators in ``tests/workloads.py``, which hold none of the method's arithmetic.

Every function restates the definition printed on the source pages in plain,
slow fp64 numpy (a matmul is the only library primitive used as a step). Pins
that tie each function to something other than itself live in
``tests/test_oracle_*.py``; functions without such a pin say "parity unpinned".
"""
from .alibi_ref import (  # noqa: F401
    slopes_ref, slopes_pow2_ref, distance_ref, bias_ref, softmax_rows_ref,
    attn_ref, attn_head_ref, attn_rows_ref, decode_ref, attn_bruteforce,
)
from .underflow import (  # noqa: F401
    format_thresholds, blindness_distance, expected_blindness_distance,
    underflow_fraction_by_distance, underflow_fraction_causal, underflow_fraction_data,
    log_scaled_blindness_distance,
)
from .mitigations import (  # noqa: F401
    TAU_D, recipe_distances, slopes_recipe_ref, variant_head_ref, variant_ref,
)
from .backward import (  # noqa: F401
    lse_head_ref, lse_ref, attn_backward_head_ref, attn_backward_ref,
)
