"""Seeded synthetic inputs for the MoE-layer forward.

This package only draws random numbers and encodes them in the input formats
(fp32, bf16, fp8 e4m3 with 128x128 block scales).  It contains none of the
layer's own arithmetic, so both the HIP path's tests and the CPU oracle can
consume its arrays without sharing any computation.
"""
from .gen import CONFIGS, Workload, make_workload, bf16_bits, fp8_block_quantise  # noqa: F401
