"""Seeded synthetic inputs shared by the CPU oracle tests, the GPU parity tests
and the benchmark.

This module holds no arithmetic of the quantisation method: it only draws
random numbers and rounds them to the storage types (bf16 / fp16) the
workloads are defined in.  Both the oracle side and the device side consume
exactly these arrays.
"""
from .gen import (  # noqa: F401
    LinearCase,
    AwqCase,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    linear_case,
    tiny_case,
    qkv_case,
    mlp_cases,
    lowres_case,
    awq_case,
    on_grid_case,
    lora_factors,
    device_normal_bf16,
    WORKLOADS,
)
