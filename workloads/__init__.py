"""Seeded synthetic inputs for paged-decode workloads.

This package only draws random numbers and shapes: context lengths, the
initial free-block order, Q/K/V values in their storage dtype, and the
churn choices (which sequences retire, which are forked) of the
continuous-batching workload.  It contains none of the method's arithmetic
(no allocator policy, no attention), so both the CPU oracle and the HIP
path can take their inputs from it without sharing any logic.
"""

from .configs import (  # noqa: F401
    CONFIGS,
    DecodeConfig,
    PrefixSharedConfig,
    config_by_name,
    draw_context_lengths,
    draw_free_order,
    pool_blocks_for,
)
from .values import (  # noqa: F401
    STORAGE_NUMPY,
    draw_decode_values,
    draw_normal_storage,
    storage_from_f32,
)
from .churn import choose_churn, draw_prefix_shared_plan  # noqa: F401
