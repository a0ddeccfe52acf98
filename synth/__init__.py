"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package holds only random-number generation and dtype casting of inputs:
none of the BitLinear arithmetic (masking, ternarization, quantization,
packing, accumulation) lives here.
"""
from .inputs import *  # noqa: F401,F403
