"""CPU oracle for the ternary-weight x INT8 matmul: test infrastructure only.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the benchmark's
CPU-baseline leg may import this package. It shares no code with the HIP
library or its binding and imports nothing from them.
"""

from .ternary_ref import (  # noqa: F401
    GROUP_K,
    QMAX,
    OracleError,
    packed_bytes,
    pack_ref,
    unpack_ref,
    quantize_ref,
    matmul_loops,
    matmul_int64,
    matmul_f64,
    matmul_ref,
    matmul_rows_cols,
    dequant_ref,
    forward_ref,
)
from .fused_ref import (  # noqa: F401
    rmsnorm_sumsq,
    rmsnorm_scale,
    rmsnorm_scaled_ref,
    rmsnorm_quantize_ref,
    epilogue_ref,
)
from .i8s_ref import I8_KMAX, i8s_matmul_ref, i8s_forward_ref  # noqa: F401,E402
from .bitnet_ref import absmean_ref, ternarize_ref, ternarize_pack_ref  # noqa: F401,E402
