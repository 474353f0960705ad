"""MI355X (gfx950) implementation of the Prox two-stage sparse SwiGLU FFN
decode step.

The compute lives in libprox.so (HIP kernels behind the C ABI of
include/prox.h); `free_ffn_activation_amd.prox` is its ctypes binding.
Build with `python -m free_ffn_activation_amd.build_lib`.
"""
__all__ = ["prox"]
