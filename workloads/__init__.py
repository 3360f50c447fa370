"""Seeded synthetic inputs for the sLSTM Newton forward.

This package only draws random numbers and lays them out. It is shared by the tests, the
benchmark and the smoke check; it imports neither the oracle nor the HIP library, and
neither of those imports it.
"""
from .configs import WORKLOADS, Workload, by_name  # noqa: F401
from .gen import (  # noqa: F401
    draw_layer_inputs,
    draw_preactivation_inputs,
    draw_decode_inputs,
    draw_head_inputs,
    packed_offsets,
    random_cotangents,
    random_cotangents_device,
    random_scan_operands,
    random_states,
    synth_preactivations,
    to_bf16,
    bf16_to_f64,
)
