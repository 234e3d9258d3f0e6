"""Seeded synthetic inputs shared by the tests, the bench and the oracle's callers.

This package draws random numbers and lays them out as raw block bytes,
fp32 and bf16 arrays.  It performs none of the MoE step's arithmetic (no
dequantisation, no routing, no products); both the HIP library and the CPU
oracle consume what it produces.
"""
from .gen import (  # noqa: F401
    WORKLOADS, Workload, codebook, q2k_blocks, cb2_blocks, q4k_blocks, block_bytes,
    expert_tensor, layer_weights, tokens, fp32_to_bf16_bits, hotlist,
)
