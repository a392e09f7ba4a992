"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This package holds workload descriptions and random-number recipes only. It
contains none of the attention method's arithmetic (no pooling, scoring,
tiering, quantisation or softmax), so that the oracle and the HIP path, which
both consume its tensors, share no code beyond their inputs.
"""
from .configs import CONFIGS, WorkloadConfig, get_workload  # noqa: F401
from .gen import generate, drift_step, to_bf16_bits, bf16_bits_to_f32  # noqa: F401
