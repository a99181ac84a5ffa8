"""Seeded synthetic inputs for the KDA core (shared by tests, smoke and bench).

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic: the gate (log-decay and beta) and the recurrence are
computed by whoever consumes these draws (the fp64 oracle or the HIP library).
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    KdaDraw,
    DecodeDraw,
    draw_prefill,
    draw_config,
    draw_decode_params,
    draw_decode_step,
    draw_alog_per_channel,
    varlen_lengths,
    orthonormal_keys_pm_quarter,
)
