"""Float64 CPU oracle for the calibration-Hessian hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test-suite, the package-level smoke
check in ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library and imports
nothing from it.

Every function here is pinned by ``tests/test_oracle.py`` against facts that
do not come from the oracle itself (exact rational brute force, the pages'
worked example, hand-derived closed forms, library routines on special cases).
"""

from .hess_oracle import (  # noqa: F401
    GramAccumulator,
    decode_bf16,
    exact_float64,
    gram_entries,
    gram_exact_fraction,
    grouped_grams,
    local_blocks,
    materialize,
    column_sum_squares,
    round_to_bf16,
    staged_values,
    chol_inverse_upper,
    quant_scale,
    gptq_quantize,
)
