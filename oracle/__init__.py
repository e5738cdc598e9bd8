"""fp64 CPU oracle for skip-softmax (BLASST) attention.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only users.  The HIP library and its
Python binding never import it, and it imports nothing from them.

Parity pins: every function here is checked in tests/test_oracle_pins.py
against closed forms, library routines, brute force and invariants that the
pages fix; see the docstring of each test for the passage it follows.
"""

from .attention import (  # noqa: F401
    MASK_COMPUTED,
    MASK_SKIPPED,
    MASK_UNVISITED,
    decode,
    dense_decode,
    dense_prefill,
    log_threshold,
    lse_combine,
    n_tiles,
    prefill,
    prefill_backward,
    skip_fraction,
    split_ranges,
    stream_pass,
    to_f64,
    visit_order,
)
from .host import factor_calibrated, factor_direct, gate_enabled, threshold  # noqa: F401
