"""Seeded synthetic inputs for one denoising iteration of block-wise dLLM decoding.

This package draws random numbers and rounds them to bf16.  It holds none of
the method's arithmetic (no attention, no softmax, no confidence, no commit
rule), so both the HIP path and the CPU oracle can consume what it produces
without sharing any computation.
"""
from .workloads import (  # noqa: F401
    Workload,
    WORKLOADS,
    get_workload,
    custom_workload,
    make_inputs,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    ROOT_SEED,
)
