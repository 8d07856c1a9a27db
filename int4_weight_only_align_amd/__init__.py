"""MI355X-native W4A16 SwiGLU Mixture-of-Experts layer (HIP kernels for gfx950 behind a C-ABI).

The binding lives in `int4_weight_only_align_amd.w4moe`; importing this package does not load the
shared library (so that it can be built first).
"""
__all__ = ["w4moe"]
