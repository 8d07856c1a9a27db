"""Seeded synthetic inputs for the W4A16 MoE layer (shared by the oracle side and the HIP side).

This package draws random numbers and lays them out in the boundary's logical formats. It holds
none of the layer's arithmetic: no unpacking, dequantisation, GEMM, activation or combine. The
router under test takes `gen_logits`; `gen_routing_softmax` draws ready-made routing (ids and
weights) for the layer's own inputs by the workload's recipe, in float32 with numpy's argsort, and
shares no code with either router implementation (the oracle's or the kernel's).
"""
from .gen import *  # noqa: F401,F403
