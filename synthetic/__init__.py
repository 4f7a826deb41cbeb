"""Seeded synthetic inputs shared by the CPU oracle's tests and the GPU path.

This package only draws random numbers and lays them out; it holds none of
the attention method's arithmetic. Both sides receive bit-identical arrays.
"""
from .gen import (  # noqa: F401
    Workload,
    WORKLOADS,
    bf16_bits,
    bf16_value,
    storage_to_f32,
    gen_W,
    gen_kv_slice,
    gen_queries,
    gen_decode_inputs,
    gen_new_tokens,
    needle_plan,
    with_overrides,
)
