"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This package draws random numbers and describes which operations a workload
issues, in which order.  It holds no part of the method itself: no pool
layout, no attention arithmetic, no allocator policy.  Both the CPU oracle and
the HIP path consume what it produces, each with its own code.
"""

from .generate import (  # noqa: F401
    Spec,
    DTYPES,
    make_spec,
    named_spec,
    scaled_spec,
    verify_spec,
    normal_bits,
    prefix_kv_bits,
    CONFIG_NAMES,
    run_flow,
    Flow,
    POISON,
    BLOCK_SIZE,
    iter_phase_chunks,
    Phase,
    step_kv_bits,
)
