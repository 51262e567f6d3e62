"""Seeded synthetic inputs shared by the tests, the bench and smoke().

This package draws random numbers and rounds them to the storage type.  It
holds none of the attention arithmetic: both the oracle and the HIP path
receive the arrays it produces and nothing else.
"""
from .workloads import (  # noqa: F401
    Workload, StackWorkload, bf16_round_f32, f32_to_bf16_bits, bf16_bits_to_f32,
    make_sla_workload, make_stack_workload, CONFIGS, config_by_name,
)
