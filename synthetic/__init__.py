"""Workload shapes and seeded synthetic inputs for the DiT block forward.

This package describes shapes and draws numbers.  It computes nothing the
method computes: no layout, no position grid, no norm, no product.  The CPU
oracle (``oracle/``) and the HIP library's tests and benchmark both take their
inputs from here and from nowhere else, which is the only thing the two sides
share.
"""

from .configs import CONFIGS, DitConfig, Modality, Segment, CondRow, get_config  # noqa: F401
from .gen import (  # noqa: F401
    fnv1a64,
    tensor_rng,
    block_weight_shapes,
    island_weight_shapes,
    block_weights,
    island_weights,
    all_weights,
    inputs,
    cond_steps,
    round_to_bf16,
    bf16_bits,
)
