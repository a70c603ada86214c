"""MX (microscaling) block quantization and block-scaled GEMM for MI355X.

The compute path lives in libmx.so (HIP kernels for gfx950 behind the C-ABI
declared in include/mx.h).  ``microscaling_block_scaled_amd.mx`` is its ctypes
binding; ``synth`` holds the seeded synthetic input generators.
"""
__all__ = ["mx", "synth"]
