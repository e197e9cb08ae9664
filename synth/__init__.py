"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws numbers: bf16 Q/K/V with outlier channels and Haar-random
orthogonal rotations.  It holds none of the method's arithmetic (no rotation,
clipping, quantization, packing or attention), so both the oracle side and the
HIP side can take their inputs from it without sharing any of the method.
"""
from .inputs import *  # noqa: F401,F403
