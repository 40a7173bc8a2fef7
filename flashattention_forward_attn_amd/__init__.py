"""MI355X (gfx950) fused attention forward: a HIP kernel library behind a C ABI.

The Python side is argument marshalling only; every step of the forward pass
runs in the HIP kernels of ``csrc/``.  Importing the package does not load the
native library; the first call does, and fails loudly if it is missing.
"""
__all__ = ["inputs"]
