"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This package only draws random numbers and lays them out in the shapes of a PBSA
decode step. It contains none of the method's arithmetic (no pooling, scoring,
softmax, selection or cache update); both the CPU oracle and the HIP library
receive its arrays as plain inputs.
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    bf16_round,
    bf16_bits,
    workload,
    make_step_inputs,
    make_dout,
    RolloutStream,
    noisy_pass,
)
