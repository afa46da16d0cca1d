"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This package only draws random numbers and rounds them to the storage dtype of
the device path; it holds none of the state-space arithmetic, so both the fp64
oracle and the HIP library can be fed from it without sharing method code.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    SELECTIVE_CONFIGS,
    SelectiveInputs,
    StepInputs,
    ForwardInputs,
    bf16_round,
    config_shapes,
    make_config_inputs,
    make_forward_inputs,
    make_selective_config_inputs,
    make_selective_inputs,
    make_step_inputs,
    round_to,
    seed_for,
)
