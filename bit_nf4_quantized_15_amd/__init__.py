"""NF4 (blocksize 64, double-quantized scales) frozen-base linear with a LoRA
branch, as hand-written HIP kernels for MI355X (gfx950) behind a C ABI.

The compute entry points live in ``bit_nf4_quantized_15_amd.qlora`` (a thin
ctypes binding over ``libqlora.so``).  Importing this package does not load the
library; importing ``qlora`` does, and fails loudly if it has not been built.
"""
__all__ = ["qlora", "workloads"]
