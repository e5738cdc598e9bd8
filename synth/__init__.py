"""Seeded synthetic inputs for skip-softmax attention.

This package only draws random numbers and lays them out as tensors.  It holds
none of the attention arithmetic, so both the CPU oracle (through the tests)
and the HIP library (through the tests and the benchmark) can take their
inputs from here without sharing any part of the method.
"""

from .generators import (  # noqa: F401
    paged_decode,
    bf16_round,
    clustered_decode,
    clustered_prefill,
    gumbel_decode,
    output_gradient,
    video_dit_field,
)
from .workloads import WORKLOADS, Workload, make_inputs  # noqa: F401
