"""Seeded synthetic workloads shared by the tests, the bench and the smoke check."""
from .configs import ALL, Config, DECODE_32K, PREFILL_128K, PREFILL_1M, RAGGED_DECODE, TINY_PREFILL, scaled
from .gen import Inputs, make_inputs, sample_rows, rope_inplace, orthonormal_projection, torch_dtype
