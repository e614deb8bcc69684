"""ctypes loader for libq4k.so -- the C ABI declared in include/q4k.h and include/w8a8.h.

The library is looked up in ``$LIBQ4K_PATH`` (a file path), then next to this
file.  If it cannot be loaded, every call raises ``Q4KLibraryError``: there is
no fallback implementation of any entry point.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_PATH = os.path.join(HERE, "libq4k.so")

# Return codes (include/q4k.h).
Q4K_OK = 0
Q4K_ERR_INVALID_ARG = -1
Q4K_ERR_ALIGN = -2
Q4K_ERR_DEVICE = -3
Q4K_ERR_LAUNCH = -4
Q4K_QK = 256
Q4K_BLOCK_BYTES = 144
Q4K_GEMV_MAX_M = 32
Q4K_MAX_N = 2147418111
Q4K_GEMM_MAX_K = 16777216
Q4K_NOALLOC_MAX_D_FF = 65536
Q4K_LAYERS_MAX = 32
Q4K_LAYERS_MAX_K = 16384
Q5K_BLOCK_BYTES = 176
Q6K_BLOCK_BYTES = 210
Q3K_BLOCK_BYTES = 110
W8A8_K_STEP = 128
W8A8_MAX_K = 130944

# Every symbol the header declares, with (restype, argtypes).
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
SIGNATURES = {
    "q4k_init": (ctypes.c_int, []),
    "q4k_device_name": (ctypes.c_char_p, []),
    "q4k_last_error": (ctypes.c_char_p, []),
    "q4k_version": (ctypes.c_int, []),
    "q4k_gemv": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "q4k_gemm": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "q4k_gemv_layers": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "q4k_swiglu_mlp": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp]),
    "q4k_swiglu_mlp_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp]),
    "q4k_dequantize_f32": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp]),
    "q4k_dequantize_bf16": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp]),
    "q4k_read_probe": (ctypes.c_int, [_vp, _i64, _vp, _vp]),
    "q5k_gemv": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "q5k_gemm": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "q5k_dequantize_f32": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp]),
    "q5k_dequantize_bf16": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp]),
    "q6k_gemv": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "q6k_dequantize_f32": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp]),
    "q6k_dequantize_bf16": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp]),
    "q3k_gemv": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "q6k_gemm": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "q3k_gemm": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "q3k_dequantize_f32": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp]),
    "q3k_dequantize_bf16": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp]),
    "w8a8_linear": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "w8a8_linear_acc": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "w8a8_dequant_epilogue": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp]),
    "w8a8_quantize_rows": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _vp]),
}


class Q4KLibraryError(RuntimeError):
    """libq4k.so could not be loaded; nothing can run without it."""


class Q4KError(RuntimeError):
    """A libq4k call returned a non-zero status."""

    def __init__(self, code: int, message: str):
        super().__init__("libq4k error %d: %s" % (code, message))
        self.code = code
        self.message = message


_lib = None
_load_error = None


def library_path() -> str:
    return os.environ.get("LIBQ4K_PATH") or DEFAULT_PATH


def load():
    """Load libq4k.so once and return the ctypes handle; raise if impossible."""
    global _lib, _load_error
    if _lib is not None:
        return _lib
    path = library_path()
    try:
        lib = ctypes.CDLL(path)
    except OSError as e:
        _load_error = "cannot load %s (%s); build it with __graft_entry__.build()" % (path, e)
        raise Q4KLibraryError(_load_error) from None
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(code: int) -> None:
    if code != Q4K_OK:
        msg = load().q4k_last_error().decode("utf-8", "replace")
        raise Q4KError(code, msg)


# Thin pass-throughs with the C names (raw device pointers as ints).
def q4k_init() -> int:
    return load().q4k_init()


def q4k_device_name() -> str:
    return load().q4k_device_name().decode()


def q4k_last_error() -> str:
    return load().q4k_last_error().decode("utf-8", "replace")


def q4k_version() -> int:
    return load().q4k_version()


def q4k_gemv(w, x, y, m, n, k, stream) -> int:
    return load().q4k_gemv(w, x, y, m, n, k, stream)


def q4k_gemv_layers(w_ptrs, x_ptrs, y_ptrs, n, k, stream) -> int:
    """w_ptrs, x_ptrs, y_ptrs: sequences of device pointers (ints), one per layer."""
    layers = len(w_ptrs)
    if not (len(x_ptrs) == len(y_ptrs) == layers):
        raise ValueError("one w, x and y pointer per layer")
    arr = ctypes.c_void_p * max(1, layers)
    return load().q4k_gemv_layers(arr(*w_ptrs), arr(*x_ptrs), arr(*y_ptrs), layers, n, k, stream)


def q4k_gemm(w, x_bf16, y, m, n, k, stream) -> int:
    return load().q4k_gemm(w, x_bf16, y, m, n, k, stream)


def q4k_swiglu_mlp(w_gate, w_up, w_down, x, h, out, d_model, d_ff, stream) -> int:
    return load().q4k_swiglu_mlp(w_gate, w_up, w_down, x, h, out, d_model, d_ff, stream)


def q4k_swiglu_mlp_noalloc(w_gate, w_up, w_down, x, out, d_model, d_ff, stream) -> int:
    return load().q4k_swiglu_mlp_noalloc(w_gate, w_up, w_down, x, out, d_model, d_ff, stream)


def q4k_dequantize_f32(w, out, n, k, stream) -> int:
    return load().q4k_dequantize_f32(w, out, n, k, stream)


def q4k_dequantize_bf16(w, out, n, k, stream) -> int:
    return load().q4k_dequantize_bf16(w, out, n, k, stream)


def q4k_read_probe(buf, nbytes, sink, stream) -> int:
    return load().q4k_read_probe(buf, nbytes, sink, stream)


def q5k_gemv(w, x, y, m, n, k, stream) -> int:
    return load().q5k_gemv(w, x, y, m, n, k, stream)


def q5k_dequantize_f32(w, out, n, k, stream) -> int:
    return load().q5k_dequantize_f32(w, out, n, k, stream)


def q5k_dequantize_bf16(w, out, n, k, stream) -> int:
    return load().q5k_dequantize_bf16(w, out, n, k, stream)


def q5k_gemm(w, x_bf16, y, m, n, k, stream) -> int:
    return load().q5k_gemm(w, x_bf16, y, m, n, k, stream)


def w8a8_linear(x, x_scale, w, w_scale, bias, out, m, n, k, stream) -> int:
    return load().w8a8_linear(x, x_scale, w, w_scale, bias, out, m, n, k, stream)


def w8a8_linear_acc(x, w, acc, m, n, k, stream) -> int:
    return load().w8a8_linear_acc(x, w, acc, m, n, k, stream)


def w8a8_dequant_epilogue(acc, out, x_scale, w_scale, bias, m, n, stream) -> int:
    return load().w8a8_dequant_epilogue(acc, out, x_scale, w_scale, bias, m, n, stream)


def w8a8_quantize_rows(x_bf16, q, scale, rows, k, stream) -> int:
    return load().w8a8_quantize_rows(x_bf16, q, scale, rows, k, stream)


def q6k_gemv(w, x, y, m, n, k, stream) -> int:
    return load().q6k_gemv(w, x, y, m, n, k, stream)


def q6k_dequantize_f32(w, out, n, k, stream) -> int:
    return load().q6k_dequantize_f32(w, out, n, k, stream)


def q6k_dequantize_bf16(w, out, n, k, stream) -> int:
    return load().q6k_dequantize_bf16(w, out, n, k, stream)


def q3k_gemv(w, x, y, m, n, k, stream) -> int:
    return load().q3k_gemv(w, x, y, m, n, k, stream)


def q3k_dequantize_f32(w, out, n, k, stream) -> int:
    return load().q3k_dequantize_f32(w, out, n, k, stream)


def q3k_dequantize_bf16(w, out, n, k, stream) -> int:
    return load().q3k_dequantize_bf16(w, out, n, k, stream)


def q6k_gemm(w, x_bf16, y, m, n, k, stream) -> int:
    return load().q6k_gemm(w, x_bf16, y, m, n, k, stream)


def q3k_gemm(w, x_bf16, y, m, n, k, stream) -> int:
    return load().q3k_gemm(w, x_bf16, y, m, n, k, stream)
