"""Ternary-weight x INT8-activation matmul for AMD MI355X (gfx950).

The BitNet-style I2_S product of the "VibeVoice-ASR-BitNet Technical Report"
(section 2.2.2): weights in {-1, 0, +1} packed 2 bits each in 128-element
groups along K with one fp32 scale per tensor, activations quantized to INT8
per token (absmax), exact int32 sums rescaled to fp32.

All work runs in libbt.so (HIP kernels for gfx950 plus host packing in C++),
declared in include/bt.h; this package only marshals arguments to it.
"""

from ._lib import LIB_PATH, BtError, lib  # noqa: F401
from .ops import (  # noqa: F401
    GEMV_MAX_M,
    GROUP_K,
    MatmulPlan,
    QuantPlan,
    RepackPlan,
    TernarizePlan,
    int8_matmul,
    int8_matmul_workspace_bytes,
    int8_repacked_bytes,
    matmul_workspace_bytes,
    new_workspace,
    pack_ternary,
    packed_bytes,
    quantize_act,
    repack_int8,
    repack_ternary,
    ternarize,
    ternarize_workspace_bytes,
    repacked_bytes,
    rmsnorm_quantize,
    ternary_matmul,
    ternary_matmul_fused,
    ternary_matmul_noalloc,
    unpack_ternary,
)
