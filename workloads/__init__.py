"""Seeded synthetic workloads shared by the tests, the bench and the oracle's callers.

This package holds only input generation (random draws, the smooth-field
recipe, rounding of the draws to the storage dtype) and the table of problem
sizes.  It contains none of the attention or selection arithmetic: the CPU
oracle (``oracle/``) and the HIP library (``dynamic_sparse_attention_dsv_amd``)
each implement that on their own.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .generator import make_inputs, bf16_bits_from_f32, f32_from_bf16_bits  # noqa: F401
