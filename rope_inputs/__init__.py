"""Seeded synthetic inputs for the rotary-embedding library's tests and benchmark.

Shared by the oracle side and the GPU side; contains random-number generators
and input structure only, never the rotary-embedding arithmetic.
"""
from .generators import BFLOAT16, SplitMix64, bfloat16_bits, normal_tensor, uniform_ints  # noqa: F401
from .workloads import EXTRA_WORKLOADS, WORKLOADS, Workload, get, mrope_ids, with_dtype, with_layout  # noqa: F401
