"""ctypes view of the plain C oracle (``q4k_oracle.c``, ``q5k_oracle.c``, ``q6k_oracle.c``,
``q3k_oracle.c``, ``w8a8_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``gemm_q4_super_block_amd``) never imports it and has no CPU fallback.

All arrays are numpy; results are fp64 (bf16 bits and int32 for the INT8 layer).  See the headers for what each
function computes and which page passage it follows.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_lib_omp = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def lib():
    """Load liboracle.so, compiling it first only if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = _declare(ctypes.CDLL(_build.LIB))
    return _lib


def lib_omp():
    """liboracle_omp.so: the same oracle with its row loops on all host cores
    (identical results); for the benchmark's all-cores CPU baseline."""
    global _lib_omp
    if _lib_omp is None:
        if not os.path.exists(_build.LIB_OMP):
            _build.build()
        _lib_omp = _declare(ctypes.CDLL(_build.LIB_OMP))
    return _lib_omp


def _pick(omp: bool):
    return lib_omp() if omp else lib()


def threads(omp: bool = False) -> int:
    """Threads the row loops of the chosen build use."""
    return _pick(omp).oracle_threads()


def _declare(L):
    """Set the ctypes signatures of every oracle entry point on a loaded build."""
    L.oracle_f16_to_f64.restype = ctypes.c_double
    L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    L.oracle_f32_to_bf16.restype = ctypes.c_uint16
    L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    L.oracle_bf16_to_f64.restype = ctypes.c_double
    L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    L.oracle_silu.restype = ctypes.c_double
    L.oracle_silu.argtypes = [ctypes.c_double]
    L.oracle_quant.restype = ctypes.c_int
    L.oracle_quant.argtypes = [_u8p, ctypes.c_int]
    L.oracle_unpack_scales.restype = None
    L.oracle_unpack_scales.argtypes = [_u8p, _u8p, _u8p]
    L.oracle_dequant_block.restype = None
    L.oracle_dequant_block.argtypes = [_u8p, _f32p]
    L.oracle_dequant_f32.argtypes = [_u8p, _i64, _i64, _f32p]
    L.oracle_dequant_bf16.argtypes = [_u8p, _i64, _i64, _u16p]
    L.oracle_gemv.argtypes = [_u8p, _f32p, _i64, _i64, _i64, _f64p, _f64p]
    L.oracle_gemv_rows.argtypes = [_u8p, _f32p, _i64, _i64, _i64, _i64p, _i64,
                                   _f64p, _f64p]
    L.oracle_gemm.argtypes = [_u8p, _u16p, _i64, _i64, _i64, _f64p, _f64p]
    L.oracle_gemm_cols.argtypes = [_u8p, _u16p, _i64, _i64, _i64, _i64p, _i64,
                                   _f64p, _f64p]
    L.oracle_swiglu_mlp.argtypes = [_u8p, _u8p, _u8p, _f32p, _i64, _i64,
                                    _f64p, _f64p, _f64p, _f64p, _f64p, _f64p,
                                    _f64p]
    L.oracle_q5k_quant.restype = ctypes.c_int
    L.oracle_q5k_quant.argtypes = [_u8p, _u8p, ctypes.c_int]
    L.oracle_q5k_dequant_block.restype = None
    L.oracle_q5k_dequant_block.argtypes = [_u8p, _f32p]
    L.oracle_q5k_dequant_f32.argtypes = [_u8p, _i64, _i64, _f32p]
    L.oracle_q5k_dequant_bf16.argtypes = [_u8p, _i64, _i64, _u16p]
    L.oracle_q5k_gemv.argtypes = [_u8p, _f32p, _i64, _i64, _i64, _f64p, _f64p]
    L.oracle_q5k_gemv_rows.argtypes = [_u8p, _f32p, _i64, _i64, _i64, _i64p, _i64,
                                       _f64p, _f64p]
    L.oracle_q5k_gemm.argtypes = [_u8p, _u16p, _i64, _i64, _i64, _f64p, _f64p]
    L.oracle_q5k_gemm_cols.argtypes = [_u8p, _u16p, _i64, _i64, _i64, _i64p, _i64,
                                       _f64p, _f64p]
    L.oracle_q3k_quant.restype = ctypes.c_int
    L.oracle_q3k_quant.argtypes = [_u8p, ctypes.c_int]
    L.oracle_q3k_scale.restype = ctypes.c_int
    L.oracle_q3k_scale.argtypes = [_u8p, ctypes.c_int]
    L.oracle_q3k_dequant_block.restype = None
    L.oracle_q3k_dequant_block.argtypes = [_u8p, _f32p]
    L.oracle_q3k_dequant_f32.argtypes = [_u8p, _i64, _i64, _f32p]
    L.oracle_q3k_dequant_bf16.argtypes = [_u8p, _i64, _i64, _u16p]
    L.oracle_q3k_gemv.argtypes = [_u8p, _f32p, _i64, _i64, _i64, _f64p, _f64p]
    L.oracle_q3k_gemv_rows.argtypes = [_u8p, _f32p, _i64, _i64, _i64, _i64p, _i64,
                                       _f64p, _f64p]
    L.oracle_q6k_quant.restype = ctypes.c_int
    L.oracle_q6k_quant.argtypes = [_u8p, ctypes.c_int]
    L.oracle_q6k_dequant_block.restype = None
    L.oracle_q6k_dequant_block.argtypes = [_u8p, _f32p]
    L.oracle_q6k_dequant_f32.argtypes = [_u8p, _i64, _i64, _f32p]
    L.oracle_q6k_dequant_bf16.argtypes = [_u8p, _i64, _i64, _u16p]
    L.oracle_q6k_gemv.argtypes = [_u8p, _f32p, _i64, _i64, _i64, _f64p, _f64p]
    L.oracle_q6k_gemv_rows.argtypes = [_u8p, _f32p, _i64, _i64, _i64, _i64p, _i64,
                                       _f64p, _f64p]
    for f in ("q6k", "q3k"):
        getattr(L, "oracle_%s_gemm" % f).argtypes = [_u8p, _u16p, _i64, _i64, _i64,
                                                     _f64p, _f64p]
        getattr(L, "oracle_%s_gemm_cols" % f).argtypes = [_u8p, _u16p, _i64, _i64, _i64,
                                                          _i64p, _i64, _f64p, _f64p]
    L.oracle_threads.restype = ctypes.c_int
    L.oracle_threads.argtypes = []
    _i8p = ctypes.POINTER(ctypes.c_int8)
    _i32p = ctypes.POINTER(ctypes.c_int32)
    L.oracle_w8a8_acc.argtypes = [_i8p, _i8p, _i64, _i64, _i64, _i32p]
    L.oracle_w8a8_epilogue.argtypes = [_i32p, _f32p, _f32p, _f32p, _i64, _i64, _u16p,
                                       _f32p]
    L.oracle_w8a8_linear.argtypes = [_i8p, _f32p, _i8p, _f32p, _f32p, _i64, _i64, _i64,
                                     _u16p]
    L.oracle_w8a8_linear_cols.argtypes = [_i8p, _f32p, _i8p, _f32p, _f32p, _i64, _i64,
                                          _i64, _i64p, _i64, _u16p]
    L.oracle_w8a8_quantize_rows.argtypes = [_u16p, _i64, _i64, _i8p, _f32p]
    for name in ("oracle_dequant_f32", "oracle_dequant_bf16", "oracle_gemv",
                 "oracle_gemv_rows", "oracle_gemm", "oracle_gemm_cols",
                 "oracle_swiglu_mlp", "oracle_q5k_dequant_f32", "oracle_q5k_dequant_bf16",
                 "oracle_q5k_gemv", "oracle_q5k_gemv_rows", "oracle_q5k_gemm",
                 "oracle_q5k_gemm_cols", "oracle_w8a8_acc", "oracle_w8a8_epilogue",
                 "oracle_w8a8_linear", "oracle_w8a8_linear_cols",
                 "oracle_w8a8_quantize_rows", "oracle_q6k_dequant_f32",
                 "oracle_q6k_dequant_bf16", "oracle_q6k_gemv", "oracle_q6k_gemv_rows",
                 "oracle_q3k_dequant_f32", "oracle_q3k_dequant_bf16", "oracle_q3k_gemv",
                 "oracle_q3k_gemv_rows", "oracle_q6k_gemm", "oracle_q6k_gemm_cols",
                 "oracle_q3k_gemm", "oracle_q3k_gemm_cols"):
        getattr(L, name).restype = ctypes.c_int
    return L


def _p(a, t):
    return a.ctypes.data_as(t)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle: %s rejected its arguments" % what)


def f16_to_f64(bits: int) -> float:
    return lib().oracle_f16_to_f64(int(bits))


def f32_to_bf16(x: float) -> int:
    return lib().oracle_f32_to_bf16(float(x))


def bf16_to_f64(bits: int) -> float:
    return lib().oracle_bf16_to_f64(int(bits))


def silu(t: float) -> float:
    return lib().oracle_silu(float(t))


def quant(qs: np.ndarray, i: int) -> int:
    qs = _c(qs, np.uint8)
    assert qs.size == 128
    return lib().oracle_quant(_p(qs, _u8p), int(i))


def unpack_scales(s: np.ndarray):
    s = _c(s, np.uint8)
    assert s.size == 12
    sc = np.zeros(8, np.uint8)
    mn = np.zeros(8, np.uint8)
    lib().oracle_unpack_scales(_p(s, _u8p), _p(sc, _u8p), _p(mn, _u8p))
    return sc, mn


def dequant_block(blk: np.ndarray) -> np.ndarray:
    blk = _c(blk, np.uint8)
    assert blk.size == 144
    w = np.zeros(256, np.float32)
    lib().oracle_dequant_block(_p(blk, _u8p), _p(w, _f32p))
    return w


def dequant_f32(w: np.ndarray, n: int, k: int) -> np.ndarray:
    w = _c(w, np.uint8)
    assert w.size == n * (k // 256) * 144
    out = np.zeros((n, k), np.float32)
    _check(lib().oracle_dequant_f32(_p(w, _u8p), n, k, _p(out, _f32p)), "dequant_f32")
    return out


def dequant_bf16(w: np.ndarray, n: int, k: int) -> np.ndarray:
    w = _c(w, np.uint8)
    assert w.size == n * (k // 256) * 144
    out = np.zeros((n, k), np.uint16)
    _check(lib().oracle_dequant_bf16(_p(w, _u8p), n, k, _p(out, _u16p)), "dequant_bf16")
    return out


def gemv(w: np.ndarray, x: np.ndarray, n: int, k: int, omp: bool = False):
    """y, a = oracle GEMV; x is fp32 [m, k] (or [k]); returns fp64 [m, n].
    omp=True runs the all-cores build (identical results)."""
    w = _c(w, np.uint8)
    x = _c(x, np.float32).reshape(-1, k)
    m = x.shape[0]
    y = np.zeros((m, n), np.float64)
    a = np.zeros((m, n), np.float64)
    _check(_pick(omp).oracle_gemv(_p(w, _u8p), _p(x, _f32p), m, n, k, _p(y, _f64p),
                                  _p(a, _f64p)), "gemv")
    return y, a


def gemv_rows(w: np.ndarray, x: np.ndarray, n: int, k: int, rows):
    """Oracle GEMV restricted to output columns ``rows``; returns [m, len(rows)]."""
    w = _c(w, np.uint8)
    x = _c(x, np.float32).reshape(-1, k)
    rows = _c(rows, np.int64)
    m = x.shape[0]
    y = np.zeros((m, rows.size), np.float64)
    a = np.zeros((m, rows.size), np.float64)
    _check(lib().oracle_gemv_rows(_p(w, _u8p), _p(x, _f32p), m, n, k, _p(rows, _i64p),
                                  rows.size, _p(y, _f64p), _p(a, _f64p)), "gemv_rows")
    return y, a


def gemm(w: np.ndarray, x_bf16: np.ndarray, n: int, k: int):
    """Y, A = oracle GEMM with X bf16 bits [m, k]; returns fp64 [m, n]."""
    w = _c(w, np.uint8)
    x = _c(x_bf16, np.uint16).reshape(-1, k)
    m = x.shape[0]
    y = np.zeros((m, n), np.float64)
    a = np.zeros((m, n), np.float64)
    _check(lib().oracle_gemm(_p(w, _u8p), _p(x, _u16p), m, n, k, _p(y, _f64p),
                             _p(a, _f64p)), "gemm")
    return y, a


def gemm_cols(w: np.ndarray, x_bf16: np.ndarray, n: int, k: int, cols, omp: bool = False):
    """Oracle GEMM restricted to output columns ``cols``; returns [m, len(cols)].
    omp=True runs the all-cores build (identical results)."""
    w = _c(w, np.uint8)
    x = _c(x_bf16, np.uint16).reshape(-1, k)
    cols = _c(cols, np.int64)
    m = x.shape[0]
    y = np.zeros((m, cols.size), np.float64)
    a = np.zeros((m, cols.size), np.float64)
    _check(_pick(omp).oracle_gemm_cols(_p(w, _u8p), _p(x, _u16p), m, n, k, _p(cols, _i64p),
                                       cols.size, _p(y, _f64p), _p(a, _f64p)), "gemm_cols")
    return y, a


def swiglu_mlp(w_gate, w_up, w_down, x, d_model: int, d_ff: int, omp: bool = False):
    """Oracle SwiGLU MLP at one token.  Returns a dict of fp64 arrays:
    g, ag, u, au, h (length d_ff) and out, aout (length d_model).
    omp=True runs the all-cores build (identical results)."""
    wg = _c(w_gate, np.uint8)
    wu = _c(w_up, np.uint8)
    wd = _c(w_down, np.uint8)
    x = _c(x, np.float32).reshape(d_model)
    r = {name: np.zeros(d_ff, np.float64) for name in ("g", "ag", "u", "au", "h")}
    r["out"] = np.zeros(d_model, np.float64)
    r["aout"] = np.zeros(d_model, np.float64)
    _check(_pick(omp).oracle_swiglu_mlp(
        _p(wg, _u8p), _p(wu, _u8p), _p(wd, _u8p), _p(x, _f32p), d_model, d_ff,
        _p(r["g"], _f64p), _p(r["ag"], _f64p), _p(r["u"], _f64p), _p(r["au"], _f64p),
        _p(r["h"], _f64p), _p(r["out"], _f64p), _p(r["aout"], _f64p)), "swiglu_mlp")
    return r


# ---- Q5_K (q5k_oracle.h) ----------------------------------------------------

Q5K_BLOCK_BYTES = 176


def q5k_quant(qh: np.ndarray, qs: np.ndarray, i: int) -> int:
    qh = _c(qh, np.uint8)
    qs = _c(qs, np.uint8)
    assert qh.size == 32 and qs.size == 128
    return lib().oracle_q5k_quant(_p(qh, _u8p), _p(qs, _u8p), int(i))


def q5k_dequant_block(blk: np.ndarray) -> np.ndarray:
    blk = _c(blk, np.uint8)
    assert blk.size == Q5K_BLOCK_BYTES
    w = np.zeros(256, np.float32)
    lib().oracle_q5k_dequant_block(_p(blk, _u8p), _p(w, _f32p))
    return w


def q5k_dequant_f32(w: np.ndarray, n: int, k: int) -> np.ndarray:
    w = _c(w, np.uint8)
    assert w.size == n * (k // 256) * Q5K_BLOCK_BYTES
    out = np.zeros((n, k), np.float32)
    _check(lib().oracle_q5k_dequant_f32(_p(w, _u8p), n, k, _p(out, _f32p)), "q5k_dequant_f32")
    return out


def q5k_dequant_bf16(w: np.ndarray, n: int, k: int) -> np.ndarray:
    w = _c(w, np.uint8)
    assert w.size == n * (k // 256) * Q5K_BLOCK_BYTES
    out = np.zeros((n, k), np.uint16)
    _check(lib().oracle_q5k_dequant_bf16(_p(w, _u8p), n, k, _p(out, _u16p)), "q5k_dequant_bf16")
    return out


def q5k_gemv(w: np.ndarray, x: np.ndarray, n: int, k: int):
    """y, a = oracle GEMV on Q5_K weights; x fp32 [m, k] (or [k]); fp64 [m, n]."""
    w = _c(w, np.uint8)
    x = _c(x, np.float32).reshape(-1, k)
    m = x.shape[0]
    y = np.zeros((m, n), np.float64)
    a = np.zeros((m, n), np.float64)
    _check(lib().oracle_q5k_gemv(_p(w, _u8p), _p(x, _f32p), m, n, k, _p(y, _f64p),
                                 _p(a, _f64p)), "q5k_gemv")
    return y, a


def q5k_gemv_rows(w: np.ndarray, x: np.ndarray, n: int, k: int, rows):
    w = _c(w, np.uint8)
    x = _c(x, np.float32).reshape(-1, k)
    rows = _c(rows, np.int64)
    m = x.shape[0]
    y = np.zeros((m, rows.size), np.float64)
    a = np.zeros((m, rows.size), np.float64)
    _check(lib().oracle_q5k_gemv_rows(_p(w, _u8p), _p(x, _f32p), m, n, k, _p(rows, _i64p),
                                      rows.size, _p(y, _f64p), _p(a, _f64p)), "q5k_gemv_rows")
    return y, a


def q5k_gemm(w: np.ndarray, x_bf16: np.ndarray, n: int, k: int):
    """Y, A = oracle GEMM on Q5_K weights; x_bf16 uint16 [m, k]; fp64 [m, n]."""
    w = _c(w, np.uint8)
    x = _c(x_bf16, np.uint16).reshape(-1, k)
    m = x.shape[0]
    y = np.zeros((m, n), np.float64)
    a = np.zeros((m, n), np.float64)
    _check(lib().oracle_q5k_gemm(_p(w, _u8p), _p(x, _u16p), m, n, k, _p(y, _f64p),
                                 _p(a, _f64p)), "q5k_gemm")
    return y, a


def q5k_gemm_cols(w: np.ndarray, x_bf16: np.ndarray, n: int, k: int, cols):
    w = _c(w, np.uint8)
    x = _c(x_bf16, np.uint16).reshape(-1, k)
    cols = _c(cols, np.int64)
    m = x.shape[0]
    y = np.zeros((m, cols.size), np.float64)
    a = np.zeros((m, cols.size), np.float64)
    _check(lib().oracle_q5k_gemm_cols(_p(w, _u8p), _p(x, _u16p), m, n, k, _p(cols, _i64p),
                                      cols.size, _p(y, _f64p), _p(a, _f64p)), "q5k_gemm_cols")
    return y, a


# ---- INT8 W8A8 linear (w8a8_oracle.h) --------------------------------------

_i8p = ctypes.POINTER(ctypes.c_int8)
_i32p = ctypes.POINTER(ctypes.c_int32)


def w8a8_acc(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """int32 [m, n] = x int8 [m, k] . w int8 [n, k]^T, exact."""
    x = _c(x, np.int8)
    w = _c(w, np.int8)
    m, k = x.shape
    n = w.shape[0]
    acc = np.zeros((m, n), np.int32)
    _check(lib().oracle_w8a8_acc(_p(x, _i8p), _p(w, _i8p), m, n, k, _p(acc, _i32p)), "w8a8_acc")
    return acc


def w8a8_epilogue(acc, x_scale, w_scale, bias=None):
    """bf16 bits [m, n] and the fp32 value before rounding, for given accumulators."""
    acc = _c(acc, np.int32)
    m, n = acc.shape
    xs = _c(x_scale, np.float32)
    ws = _c(w_scale, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    out = np.zeros((m, n), np.uint16)
    f = np.zeros((m, n), np.float32)
    _check(lib().oracle_w8a8_epilogue(_p(acc, _i32p), _p(xs, _f32p), _p(ws, _f32p),
                                      None if b is None else _p(b, _f32p), m, n,
                                      _p(out, _u16p), _p(f, _f32p)), "w8a8_epilogue")
    return out, f


def w8a8_linear(x, x_scale, w, w_scale, bias=None) -> np.ndarray:
    """bf16 bits [m, n] of the W8A8 linear layer (acc then the epilogue)."""
    x = _c(x, np.int8)
    w = _c(w, np.int8)
    m, k = x.shape
    n = w.shape[0]
    xs = _c(x_scale, np.float32)
    ws = _c(w_scale, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    out = np.zeros((m, n), np.uint16)
    _check(lib().oracle_w8a8_linear(_p(x, _i8p), _p(xs, _f32p), _p(w, _i8p), _p(ws, _f32p),
                                    None if b is None else _p(b, _f32p), m, n, k,
                                    _p(out, _u16p)), "w8a8_linear")
    return out


def w8a8_linear_cols(x, x_scale, w, w_scale, bias, cols) -> np.ndarray:
    """bf16 bits [m, len(cols)]: the W8A8 linear layer at the given output columns."""
    x = _c(x, np.int8)
    w = _c(w, np.int8)
    m, k = x.shape
    n = w.shape[0]
    xs = _c(x_scale, np.float32)
    ws = _c(w_scale, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    cols = _c(cols, np.int64)
    out = np.zeros((m, len(cols)), np.uint16)
    _check(lib().oracle_w8a8_linear_cols(_p(x, _i8p), _p(xs, _f32p), _p(w, _i8p),
                                         _p(ws, _f32p), None if b is None else _p(b, _f32p),
                                         m, n, k, _p(cols, _i64p), len(cols), _p(out, _u16p)),
           "w8a8_linear_cols")
    return out


def w8a8_quantize_rows(x_bf16_bits):
    """Row quantizer: bf16 bits [rows, k] -> (int8 codes [rows, k], fp32 scales [rows])."""
    x = _c(x_bf16_bits, np.uint16)
    rows, k = x.shape
    q = np.zeros((rows, k), np.int8)
    s = np.zeros(rows, np.float32)
    _check(lib().oracle_w8a8_quantize_rows(_p(x, _u16p), rows, k, _p(q, _i8p), _p(s, _f32p)),
           "w8a8_quantize_rows")
    return q, s


# ---- Q6_K (q6k_oracle.h) ----------------------------------------------------

Q6K_BLOCK_BYTES = 210


def q6k_quant(blk: np.ndarray, i: int) -> int:
    blk = _c(blk, np.uint8)
    assert blk.size == Q6K_BLOCK_BYTES
    return lib().oracle_q6k_quant(_p(blk, _u8p), int(i))


def q6k_dequant_block(blk: np.ndarray) -> np.ndarray:
    blk = _c(blk, np.uint8)
    assert blk.size == Q6K_BLOCK_BYTES
    w = np.zeros(256, np.float32)
    lib().oracle_q6k_dequant_block(_p(blk, _u8p), _p(w, _f32p))
    return w


def q6k_dequant_f32(w: np.ndarray, n: int, k: int) -> np.ndarray:
    w = _c(w, np.uint8)
    assert w.size == n * (k // 256) * Q6K_BLOCK_BYTES
    out = np.zeros((n, k), np.float32)
    _check(lib().oracle_q6k_dequant_f32(_p(w, _u8p), n, k, _p(out, _f32p)), "q6k_dequant_f32")
    return out


def q6k_dequant_bf16(w: np.ndarray, n: int, k: int) -> np.ndarray:
    w = _c(w, np.uint8)
    assert w.size == n * (k // 256) * Q6K_BLOCK_BYTES
    out = np.zeros((n, k), np.uint16)
    _check(lib().oracle_q6k_dequant_bf16(_p(w, _u8p), n, k, _p(out, _u16p)), "q6k_dequant_bf16")
    return out


def q6k_gemv(w: np.ndarray, x: np.ndarray, n: int, k: int):
    """y, a = oracle GEMV on Q6_K weights; x fp32 [m, k] (or [k]); fp64 [m, n]."""
    w = _c(w, np.uint8)
    x = _c(x, np.float32).reshape(-1, k)
    m = x.shape[0]
    y = np.zeros((m, n), np.float64)
    a = np.zeros((m, n), np.float64)
    _check(lib().oracle_q6k_gemv(_p(w, _u8p), _p(x, _f32p), m, n, k, _p(y, _f64p),
                                 _p(a, _f64p)), "q6k_gemv")
    return y, a


def q6k_gemv_rows(w: np.ndarray, x: np.ndarray, n: int, k: int, rows):
    w = _c(w, np.uint8)
    x = _c(x, np.float32).reshape(-1, k)
    rows = _c(rows, np.int64)
    m = x.shape[0]
    y = np.zeros((m, rows.size), np.float64)
    a = np.zeros((m, rows.size), np.float64)
    _check(lib().oracle_q6k_gemv_rows(_p(w, _u8p), _p(x, _f32p), m, n, k, _p(rows, _i64p),
                                      rows.size, _p(y, _f64p), _p(a, _f64p)), "q6k_gemv_rows")
    return y, a


def q6k_gemm(w: np.ndarray, x_bf16: np.ndarray, n: int, k: int):
    """Y, A = oracle GEMM on Q6_K weights; x_bf16 uint16 [m, k]; fp64 [m, n]."""
    w = _c(w, np.uint8)
    assert w.size == n * (k // 256) * Q6K_BLOCK_BYTES
    x = _c(x_bf16, np.uint16).reshape(-1, k)
    m = x.shape[0]
    y = np.zeros((m, n), np.float64)
    a = np.zeros((m, n), np.float64)
    _check(lib().oracle_q6k_gemm(_p(w, _u8p), _p(x, _u16p), m, n, k, _p(y, _f64p),
                                 _p(a, _f64p)), "q6k_gemm")
    return y, a


def q6k_gemm_cols(w: np.ndarray, x_bf16: np.ndarray, n: int, k: int, cols):
    """Oracle Q6_K GEMM at output columns ``cols``; returns [m, len(cols)]."""
    w = _c(w, np.uint8)
    assert w.size == n * (k // 256) * Q6K_BLOCK_BYTES
    x = _c(x_bf16, np.uint16).reshape(-1, k)
    cols = _c(cols, np.int64)
    m = x.shape[0]
    y = np.zeros((m, cols.size), np.float64)
    a = np.zeros((m, cols.size), np.float64)
    _check(lib().oracle_q6k_gemm_cols(_p(w, _u8p), _p(x, _u16p), m, n, k, _p(cols, _i64p),
                                      cols.size, _p(y, _f64p), _p(a, _f64p)), "q6k_gemm_cols")
    return y, a


# ---- Q3_K (q3k_oracle.h) ----------------------------------------------------

Q3K_BLOCK_BYTES = 110


def q3k_quant(blk: np.ndarray, i: int) -> int:
    blk = _c(blk, np.uint8)
    assert blk.size == Q3K_BLOCK_BYTES
    return lib().oracle_q3k_quant(_p(blk, _u8p), int(i))


def q3k_scale(blk: np.ndarray, t: int) -> int:
    blk = _c(blk, np.uint8)
    assert blk.size == Q3K_BLOCK_BYTES
    return lib().oracle_q3k_scale(_p(blk, _u8p), int(t))


def q3k_dequant_block(blk: np.ndarray) -> np.ndarray:
    blk = _c(blk, np.uint8)
    assert blk.size == Q3K_BLOCK_BYTES
    w = np.zeros(256, np.float32)
    lib().oracle_q3k_dequant_block(_p(blk, _u8p), _p(w, _f32p))
    return w


def q3k_dequant_f32(w: np.ndarray, n: int, k: int) -> np.ndarray:
    w = _c(w, np.uint8)
    assert w.size == n * (k // 256) * Q3K_BLOCK_BYTES
    out = np.zeros((n, k), np.float32)
    _check(lib().oracle_q3k_dequant_f32(_p(w, _u8p), n, k, _p(out, _f32p)), "q3k_dequant_f32")
    return out


def q3k_dequant_bf16(w: np.ndarray, n: int, k: int) -> np.ndarray:
    w = _c(w, np.uint8)
    assert w.size == n * (k // 256) * Q3K_BLOCK_BYTES
    out = np.zeros((n, k), np.uint16)
    _check(lib().oracle_q3k_dequant_bf16(_p(w, _u8p), n, k, _p(out, _u16p)), "q3k_dequant_bf16")
    return out


def q3k_gemv(w: np.ndarray, x: np.ndarray, n: int, k: int):
    """y, a = oracle GEMV on Q3_K weights; x fp32 [m, k] (or [k]); fp64 [m, n]."""
    w = _c(w, np.uint8)
    x = _c(x, np.float32).reshape(-1, k)
    m = x.shape[0]
    y = np.zeros((m, n), np.float64)
    a = np.zeros((m, n), np.float64)
    _check(lib().oracle_q3k_gemv(_p(w, _u8p), _p(x, _f32p), m, n, k, _p(y, _f64p),
                                 _p(a, _f64p)), "q3k_gemv")
    return y, a


def q3k_gemv_rows(w: np.ndarray, x: np.ndarray, n: int, k: int, rows):
    w = _c(w, np.uint8)
    x = _c(x, np.float32).reshape(-1, k)
    rows = _c(rows, np.int64)
    m = x.shape[0]
    y = np.zeros((m, rows.size), np.float64)
    a = np.zeros((m, rows.size), np.float64)
    _check(lib().oracle_q3k_gemv_rows(_p(w, _u8p), _p(x, _f32p), m, n, k, _p(rows, _i64p),
                                      rows.size, _p(y, _f64p), _p(a, _f64p)), "q3k_gemv_rows")
    return y, a


def q3k_gemm(w: np.ndarray, x_bf16: np.ndarray, n: int, k: int):
    """Y, A = oracle GEMM on Q3_K weights; x_bf16 uint16 [m, k]; fp64 [m, n]."""
    w = _c(w, np.uint8)
    assert w.size == n * (k // 256) * Q3K_BLOCK_BYTES
    x = _c(x_bf16, np.uint16).reshape(-1, k)
    m = x.shape[0]
    y = np.zeros((m, n), np.float64)
    a = np.zeros((m, n), np.float64)
    _check(lib().oracle_q3k_gemm(_p(w, _u8p), _p(x, _u16p), m, n, k, _p(y, _f64p),
                                 _p(a, _f64p)), "q3k_gemm")
    return y, a


def q3k_gemm_cols(w: np.ndarray, x_bf16: np.ndarray, n: int, k: int, cols):
    """Oracle Q3_K GEMM at output columns ``cols``; returns [m, len(cols)]."""
    w = _c(w, np.uint8)
    assert w.size == n * (k // 256) * Q3K_BLOCK_BYTES
    x = _c(x_bf16, np.uint16).reshape(-1, k)
    cols = _c(cols, np.int64)
    m = x.shape[0]
    y = np.zeros((m, cols.size), np.float64)
    a = np.zeros((m, cols.size), np.float64)
    _check(lib().oracle_q3k_gemm_cols(_p(w, _u8p), _p(x, _u16p), m, n, k, _p(cols, _i64p),
                                      cols.size, _p(y, _f64p), _p(a, _f64p)), "q3k_gemm_cols")
    return y, a
