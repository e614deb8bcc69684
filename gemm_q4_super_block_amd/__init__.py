"""libq4k: the Q4_K linear layer on AMD MI355X (gfx950), with its Q5_K, Q6_K, Q3_K and INT8 W8A8 siblings.

The compute lives in ``libq4k.so`` (hand-written HIP kernels behind a C ABI,
``include/q4k.h`` and ``include/w8a8.h``); this package only loads it and marshals
torch tensors.
"""
from ._lib import Q4KError, Q4KLibraryError, load as load_library  # noqa: F401
from .ops import (dequantize_bf16, dequantize_f32, gemm, gemv, gemv_layers, q3k_dequantize_bf16,  # noqa: F401
                  q3k_dequantize_f32, q3k_gemm, q3k_gemv, q5k_dequantize_bf16,
                  prepare_weight, q5k_dequantize_f32, q5k_gemm, q5k_gemv, q6k_dequantize_bf16,
                  q6k_dequantize_f32, q6k_gemm, q6k_gemv, swiglu_mlp, swiglu_mlp_noalloc,
                  w8a8_dequant, w8a8_linear, w8a8_linear_acc, w8a8_quantize_rows)

__all__ = ["gemv", "gemv_layers", "gemm", "swiglu_mlp", "swiglu_mlp_noalloc", "dequantize_f32", "dequantize_bf16",
           "q5k_gemv", "q5k_gemm", "q5k_dequantize_f32", "q5k_dequantize_bf16",
           "q6k_gemv", "q6k_gemm", "q6k_dequantize_f32", "q6k_dequantize_bf16",
           "q3k_gemv", "q3k_gemm", "q3k_dequantize_f32", "q3k_dequantize_bf16",
           "w8a8_linear", "w8a8_linear_acc", "w8a8_dequant", "w8a8_quantize_rows",
           "prepare_weight", "Q4KError", "Q4KLibraryError", "load_library"]
