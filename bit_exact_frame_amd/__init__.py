"""bit_exact_frame_amd: bit-exact float_moment / float_psnr frame reductions
on MI355X (gfx950).

The computation lives in the HIP library ``libbef.so`` behind the C ABI of
``include/bef.h``; ``bit_exact_frame_amd.api`` is its thin ctypes binding.
Importing this package loads nothing native; ``synth`` (seeded inputs) is
usable without a GPU.
"""
__all__ = ["synth"]
