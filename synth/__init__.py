"""Seeded synthetic workloads for the Finch WKV pre-fill.

This module only draws random numbers and rounds them to the storage type; it
holds none of the WKV arithmetic.  Both the oracle tests and the GPU tests (and
the benchmark) take their inputs from here, so the two sides see bit-identical
values.
"""
from .configs import CONFIGS, WorkloadConfig, get_config  # noqa: F401
from .gen import (Workload, make_workload, f32_to_bf16_bits,  # noqa: F401
                  bf16_bits_to_f32, random_slice, select_heads, make_norm_inputs,
                  make_compress_inputs)
from .compare import block_errors, max_block_error, error_report  # noqa: F401
