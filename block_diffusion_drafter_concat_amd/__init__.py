"""MI355X-native drafter hot path of block-diffusion speculative decoding.

The compute lives in ``libdflash.so`` (hand-written HIP for gfx950) behind a
C ABI declared in ``include/dflash.h``; ``block_diffusion_drafter_concat_amd.lib``
is its thin ctypes binding.  Importing this package loads nothing; the binding
loads the library on first use and raises if it is missing.
"""
__all__ = ["configs", "synth"]
