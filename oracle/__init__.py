"""Float64 CPU oracle for the sLSTM (mix='diag') Newton forward.

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the benchmark's
CPU-baseline leg. The product path never imports it.
"""
from . import slstm_ref, lanes  # noqa: F401
