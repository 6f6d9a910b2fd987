"""MI355X-native implicit-GEMM 2-D convolution: forward, d_input and wgrad.

The compute path is the C-ABI library ``libgc.so`` (hand-written HIP for
gfx950, declared in ``include/gc.h``); :mod:`backward_implicit_gemm_amd.binding`
marshals torch tensors into its calls.  Importing this package loads nothing;
the binding loads the library on first use and raises if it is missing.
"""
__all__ = ["binding", "inputs"]
