"""MI355X-native sLSTM (mix='diag') forward: Newton-parallel solve and sequential steps,
hand-written HIP for gfx950 behind a C ABI (include/slstm.h), with this thin ctypes binding.
"""
from .slstm import (  # noqa: F401
    NewtonDivergenceError,
    NewtonStats,
    SlstmError,
    input_projection,
    load,
    newton_forward,
    newton_workspace_bytes,
    read_stats,
    residual_jacobian,
    scan_block4,
    sequential_forward,
    warm_start,
)
