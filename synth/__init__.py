"""Seeded synthetic inputs shaped like the 1.5B, 28-layer decoder's linear layers.

This package only draws random numbers. It holds none of the method's
arithmetic (no packing, quantization or matmul), so the oracle and the HIP
path can both consume the same bytes without sharing any of the computation.
"""

from .generators import (  # noqa: F401
    PROJECTIONS,
    N_LAYERS,
    HIDDEN,
    config0,
    decode_problem,
    decode_remainder_problem,
    prefill_problem,
    long_prefill_problem,
    ternary_weights,
    projection_rng,
    small_problem,
    device_student_t3,
    fp_weights,
    device_fp_weights,
    CFG_LONG,
    REMAINDER_MS,
)
