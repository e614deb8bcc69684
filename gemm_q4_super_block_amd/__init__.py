"""libq4k: the Q4_K linear layer on AMD MI355X (gfx950).

The compute lives in ``libq4k.so`` (hand-written HIP kernels behind a C ABI,
``include/q4k.h``); this package only loads it and marshals torch tensors.
"""
from ._lib import Q4KError, Q4KLibraryError, load as load_library  # noqa: F401
from .ops import (dequantize_bf16, dequantize_f32, gemm, gemv, q5k_dequantize_bf16,  # noqa: F401
                  q5k_dequantize_f32, q5k_gemm, q5k_gemv, swiglu_mlp)

__all__ = ["gemv", "gemm", "swiglu_mlp", "dequantize_f32", "dequantize_bf16",
           "Q4KError", "Q4KLibraryError", "load_library"]
