"""libdblock: one denoising iteration of block-wise diffusion-LLM decoding on MI355X.

The compute lives in ``libdblock.so`` (hand-written HIP for gfx950, C ABI in
``include/dblock.h``).  ``block_wise_decoding_amd.dblock`` is a thin ctypes
binding with the same entry-point names; importing this package does not load
the library.
"""
__all__ = ["dblock", "build"]
