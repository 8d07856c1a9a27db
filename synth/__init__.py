"""Seeded synthetic inputs for the W4A16 MoE layer (shared by the oracle side and the HIP side).

This package draws random numbers and lays them out in the boundary's logical formats. It holds
none of the layer's arithmetic: no unpacking, dequantisation, GEMM, activation or combine.
"""
from .gen import *  # noqa: F401,F403
