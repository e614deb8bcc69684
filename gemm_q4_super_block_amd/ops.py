"""torch-facing wrappers over the libq4k C ABI (argument marshalling only).

PyTorch provides device memory and the current stream; every computation runs
in libq4k's HIP kernels.  Weights are ``torch.uint8`` tensors holding raw Q4_K
super-blocks, shape ``[n, (k // 256) * 144]`` (Q5_K: 176-byte blocks,
``[n, (k // 256) * 176]``, for the ``q5k_`` functions; Q6_K: 210-byte blocks for the
``q6k_`` functions; Q3_K: 110-byte blocks for the ``q3k_`` functions).  The INT8 W8A8 layer
(``w8a8_*``) takes int8 codes with fp32 per-row scales and returns bf16.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import Q3K_BLOCK_BYTES, Q4K_BLOCK_BYTES, Q4K_QK, Q5K_BLOCK_BYTES, Q6K_BLOCK_BYTES, check


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _q4k_shape(w: torch.Tensor, block: int = Q4K_BLOCK_BYTES):
    if w.dtype != torch.uint8 or w.dim() != 2 or not w.is_cuda or not w.is_contiguous():
        raise ValueError("weights must be a contiguous CUDA uint8 tensor [n, k/256*%d]" % block)
    n, row_bytes = w.shape
    if row_bytes % block:
        raise ValueError("row length %d is not a whole number of %d-byte blocks"
                         % (row_bytes, block))
    return n, (row_bytes // block) * Q4K_QK


def _dev_tensor(t: torch.Tensor, dtype, what: str) -> torch.Tensor:
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous CUDA %s tensor" % (what, dtype))
    return t


def _out_tensor(t: torch.Tensor, dtype, shape, device: torch.device, what: str) -> torch.Tensor:
    """A caller-supplied output: dtype, contiguity, exact shape and device are
    checked before the kernels get its pointer (a short buffer would be
    written past its end)."""
    _dev_tensor(t, dtype, what)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (what, tuple(t.shape), tuple(shape)))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (what, t.device, device))
    return t


def _same_device(device: torch.device, *named):
    for what, t in named:
        if t.device != device:
            raise ValueError("%s is on %s, expected %s" % (what, t.device, device))


def gemv(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """y = x W^T for fp32 x [k] or [m, k] (m <= 32); returns fp32 [n] or [m, n]."""
    return _gemv(w, x, out, Q4K_BLOCK_BYTES, _lib.q4k_gemv)


def q5k_gemv(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """gemv() for a Q5_K W (uint8 [n, k/256*176])."""
    return _gemv(w, x, out, Q5K_BLOCK_BYTES, _lib.q5k_gemv)


def q6k_gemv(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """gemv() for a Q6_K W (uint8 [n, k/256*210])."""
    return _gemv(w, x, out, Q6K_BLOCK_BYTES, _lib.q6k_gemv)


def q3k_gemv(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """gemv() for a Q3_K W (uint8 [n, k/256*110])."""
    return _gemv(w, x, out, Q3K_BLOCK_BYTES, _lib.q3k_gemv)


def _gemv(w, x, out, block, fn):
    n, k = _q4k_shape(w, block)
    _dev_tensor(x, torch.float32, "x")
    _same_device(w.device, ("x", x))
    squeeze = x.dim() == 1
    x2 = x.view(1, -1) if squeeze else x
    if x2.dim() != 2 or x2.shape[1] != k:
        raise ValueError("x has shape %s, expected [..., %d]" % (tuple(x.shape), k))
    m = x2.shape[0]
    shape = (n,) if squeeze else (m, n)
    y = out if out is not None else torch.empty(shape, dtype=torch.float32, device=w.device)
    _out_tensor(y, torch.float32, shape, w.device, "out")
    check(fn(w.data_ptr(), x2.data_ptr(), y.data_ptr(), m, n, k, _stream(w.device)))
    return y


def gemv_layers(ws, xs, outs=None):
    """Independent batch-1 GEMVs of one shape in one launch: y[l] = W[l] x[l]
    for lists of Q4_K weights [n, k/256*144] and fp32 x [k]; returns the list
    of fp32 y [n]."""
    if not ws or len(ws) != len(xs) or (outs is not None and len(outs) != len(ws)):
        raise ValueError("one weight, x (and out) per layer")
    n, k = _q4k_shape(ws[0])
    dev = ws[0].device
    for l, (w, x) in enumerate(zip(ws, xs)):
        if _q4k_shape(w) != (n, k):
            raise ValueError("layer %d: every weight must be [%d, %d]" % (l, n, k))
        _dev_tensor(x, torch.float32, "x[%d]" % l)
        _same_device(dev, ("w[%d]" % l, w), ("x[%d]" % l, x))
        if x.dim() != 1 or x.shape[0] != k:
            raise ValueError("x[%d] must be [%d]" % (l, k))
    ys = outs if outs is not None else [torch.empty(n, dtype=torch.float32, device=dev) for _ in ws]
    for l, y in enumerate(ys):
        _out_tensor(y, torch.float32, (n,), dev, "out[%d]" % l)
    check(_lib.q4k_gemv_layers([w.data_ptr() for w in ws], [x.data_ptr() for x in xs],
                               [y.data_ptr() for y in ys], n, k, _stream(dev)))
    return ys


def gemm(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X W^T for bf16 X [m, k]; returns fp32 [m, n]."""
    return _gemm(w, x, out, Q4K_BLOCK_BYTES, _lib.q4k_gemm)


def q5k_gemm(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """gemm() for a Q5_K W (uint8 [n, k/256*176])."""
    return _gemm(w, x, out, Q5K_BLOCK_BYTES, _lib.q5k_gemm)


def q6k_gemm(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """gemm() for a Q6_K W (uint8 [n, k/256*210])."""
    return _gemm(w, x, out, Q6K_BLOCK_BYTES, _lib.q6k_gemm)


def q3k_gemm(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """gemm() for a Q3_K W (uint8 [n, k/256*110])."""
    return _gemm(w, x, out, Q3K_BLOCK_BYTES, _lib.q3k_gemm)


def _gemm(w, x, out, block, fn):
    n, k = _q4k_shape(w, block)
    _dev_tensor(x, torch.bfloat16, "x")
    _same_device(w.device, ("x", x))
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x has shape %s, expected [m, %d]" % (tuple(x.shape), k))
    m = x.shape[0]
    y = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=w.device)
    _out_tensor(y, torch.float32, (m, n), w.device, "out")
    check(fn(w.data_ptr(), x.data_ptr(), y.data_ptr(), m, n, k, _stream(w.device)))
    return y


def swiglu_mlp(w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
               x: torch.Tensor, h: torch.Tensor | None = None,
               out: torch.Tensor | None = None):
    """out = W_down (silu(W_gate x) * (W_up x)) at one token; returns (out, h)."""
    d_ff, d_model = _q4k_shape(w_gate)
    if _q4k_shape(w_up) != (d_ff, d_model) or _q4k_shape(w_down) != (d_model, d_ff):
        raise ValueError("gate/up must be [d_ff, d_model] and down [d_model, d_ff]")
    _dev_tensor(x, torch.float32, "x")
    _same_device(w_gate.device, ("w_up", w_up), ("w_down", w_down), ("x", x))
    if x.dim() != 1 or x.numel() != d_model:
        raise ValueError("x must be [d_model = %d]" % d_model)
    if h is None:
        h = torch.empty(d_ff, dtype=torch.float32, device=x.device)
    if out is None:
        out = torch.empty(d_model, dtype=torch.float32, device=x.device)
    _out_tensor(h, torch.float32, (d_ff,), x.device, "h")
    _out_tensor(out, torch.float32, (d_model,), x.device, "out")
    check(_lib.q4k_swiglu_mlp(w_gate.data_ptr(), w_up.data_ptr(), w_down.data_ptr(),
                              x.data_ptr(), h.data_ptr(), out.data_ptr(), d_model, d_ff,
                              _stream(x.device)))
    return out, h


def swiglu_mlp_noalloc(w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                       x: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """swiglu_mlp() with h in the library's device scratch: the entry point
    allocates nothing, and `out` [d_model] is the caller's (so a call under
    graph capture allocates nothing either).  Calls that overlap on one GPU
    share the scratch and race."""
    d_ff, d_model = _q4k_shape(w_gate)
    if _q4k_shape(w_up) != (d_ff, d_model) or _q4k_shape(w_down) != (d_model, d_ff):
        raise ValueError("gate/up must be [d_ff, d_model] and down [d_model, d_ff]")
    _dev_tensor(x, torch.float32, "x")
    _same_device(w_gate.device, ("w_up", w_up), ("w_down", w_down), ("x", x))
    if x.dim() != 1 or x.numel() != d_model:
        raise ValueError("x must be [d_model = %d]" % d_model)
    _out_tensor(out, torch.float32, (d_model,), x.device, "out")
    check(_lib.q4k_swiglu_mlp_noalloc(w_gate.data_ptr(), w_up.data_ptr(), w_down.data_ptr(),
                                      x.data_ptr(), out.data_ptr(), d_model, d_ff,
                                      _stream(x.device)))
    return out


def dequantize_f32(w: torch.Tensor) -> torch.Tensor:
    """Dequantized W as fp32 [n, k]."""
    n, k = _q4k_shape(w)
    out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    check(_lib.q4k_dequantize_f32(w.data_ptr(), out.data_ptr(), n, k, _stream(w.device)))
    return out


def dequantize_bf16(w: torch.Tensor) -> torch.Tensor:
    """Dequantized W as bf16 [n, k] (nearest-even rounding of the fp32 weight)."""
    n, k = _q4k_shape(w)
    out = torch.empty((n, k), dtype=torch.bfloat16, device=w.device)
    check(_lib.q4k_dequantize_bf16(w.data_ptr(), out.data_ptr(), n, k, _stream(w.device)))
    return out


def q5k_dequantize_f32(w: torch.Tensor) -> torch.Tensor:
    """Dequantized Q5_K W as fp32 [n, k]."""
    n, k = _q4k_shape(w, Q5K_BLOCK_BYTES)
    out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    check(_lib.q5k_dequantize_f32(w.data_ptr(), out.data_ptr(), n, k, _stream(w.device)))
    return out


def q5k_dequantize_bf16(w: torch.Tensor) -> torch.Tensor:
    """Dequantized Q5_K W as bf16 [n, k] (nearest-even rounding of the fp32 weight)."""
    n, k = _q4k_shape(w, Q5K_BLOCK_BYTES)
    out = torch.empty((n, k), dtype=torch.bfloat16, device=w.device)
    check(_lib.q5k_dequantize_bf16(w.data_ptr(), out.data_ptr(), n, k, _stream(w.device)))
    return out


def q6k_dequantize_f32(w: torch.Tensor) -> torch.Tensor:
    """Dequantized Q6_K W as fp32 [n, k]."""
    n, k = _q4k_shape(w, Q6K_BLOCK_BYTES)
    out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    check(_lib.q6k_dequantize_f32(w.data_ptr(), out.data_ptr(), n, k, _stream(w.device)))
    return out


def q6k_dequantize_bf16(w: torch.Tensor) -> torch.Tensor:
    """Dequantized Q6_K W as bf16 [n, k] (nearest-even rounding of the fp32 weight)."""
    n, k = _q4k_shape(w, Q6K_BLOCK_BYTES)
    out = torch.empty((n, k), dtype=torch.bfloat16, device=w.device)
    check(_lib.q6k_dequantize_bf16(w.data_ptr(), out.data_ptr(), n, k, _stream(w.device)))
    return out


def q3k_dequantize_f32(w: torch.Tensor) -> torch.Tensor:
    """Dequantized Q3_K W as fp32 [n, k]."""
    n, k = _q4k_shape(w, Q3K_BLOCK_BYTES)
    out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    check(_lib.q3k_dequantize_f32(w.data_ptr(), out.data_ptr(), n, k, _stream(w.device)))
    return out


def q3k_dequantize_bf16(w: torch.Tensor) -> torch.Tensor:
    """Dequantized Q3_K W as bf16 [n, k] (nearest-even rounding of the fp32 weight)."""
    n, k = _q4k_shape(w, Q3K_BLOCK_BYTES)
    out = torch.empty((n, k), dtype=torch.bfloat16, device=w.device)
    check(_lib.q3k_dequantize_bf16(w.data_ptr(), out.data_ptr(), n, k, _stream(w.device)))
    return out


# ---------------------------------------------------------------- INT8 W8A8

def _vec(t, n, what, device=None):
    _dev_tensor(t, torch.float32, what)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (what, t.device, device))
    if t.dim() != 1 or t.shape[0] != n:
        raise ValueError("%s has shape %s, expected [%d]" % (what, tuple(t.shape), n))
    return t.data_ptr()


def _w8_operands(x, w):
    _dev_tensor(x, torch.int8, "x")
    _dev_tensor(w, torch.int8, "w")
    _same_device(x.device, ("w", w))
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x [m, k] and w [n, k] expected, got %s and %s"
                         % (tuple(x.shape), tuple(w.shape)))
    return x.shape[0], w.shape[0], x.shape[1]


def w8a8_linear(x: torch.Tensor, x_scale: torch.Tensor, w: torch.Tensor, w_scale: torch.Tensor,
                bias: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 [m, n] = (x w^T) * x_scale[:, None] * w_scale[None, :] + bias, int8 x and w."""
    m, n, k = _w8_operands(x, w)
    xs = _vec(x_scale, m, "x_scale", x.device)
    ws = _vec(w_scale, n, "w_scale", x.device)
    b = None if bias is None else _vec(bias, n, "bias", x.device)
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _out_tensor(y, torch.bfloat16, (m, n), x.device, "out")
    check(_lib.w8a8_linear(x.data_ptr(), xs, w.data_ptr(), ws, b, y.data_ptr(), m, n, k,
                           _stream(x.device)))
    return y


def w8a8_linear_acc(x: torch.Tensor, w: torch.Tensor,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """int32 [m, n] = x w^T, exact, for int8 x [m, k] and w [n, k]."""
    m, n, k = _w8_operands(x, w)
    acc = out if out is not None else torch.empty((m, n), dtype=torch.int32, device=x.device)
    _out_tensor(acc, torch.int32, (m, n), x.device, "out")
    check(_lib.w8a8_linear_acc(x.data_ptr(), w.data_ptr(), acc.data_ptr(), m, n, k,
                               _stream(x.device)))
    return acc


def w8a8_dequant(acc: torch.Tensor, x_scale: torch.Tensor, w_scale: torch.Tensor,
                 bias: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """The dequant epilogue alone: int32 [m, n] -> bf16 [m, n]."""
    _dev_tensor(acc, torch.int32, "acc")
    if acc.dim() != 2:
        raise ValueError("acc must be [m, n]")
    m, n = acc.shape
    xs = _vec(x_scale, m, "x_scale", acc.device)
    ws = _vec(w_scale, n, "w_scale", acc.device)
    b = None if bias is None else _vec(bias, n, "bias", acc.device)
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=acc.device)
    _out_tensor(y, torch.bfloat16, (m, n), acc.device, "out")
    check(_lib.w8a8_dequant_epilogue(acc.data_ptr(), y.data_ptr(), xs, ws, b, m, n,
                                     _stream(acc.device)))
    return y


def w8a8_quantize_rows(x: torch.Tensor):
    """Per-row int8 quantization of bf16 [rows, k]: (int8 codes [rows, k], fp32 scales [rows])."""
    _dev_tensor(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be [rows, k]")
    rows, k = x.shape
    q = torch.empty((rows, k), dtype=torch.int8, device=x.device)
    s = torch.empty((rows,), dtype=torch.float32, device=x.device)
    check(_lib.w8a8_quantize_rows(x.data_ptr(), q.data_ptr(), s.data_ptr(), rows, k,
                                  _stream(x.device)))
    return q, s


def prepare_weight(w: torch.Tensor):
    """bf16 weight [n, k] -> (int8 [n, k], fp32 per-row scale [n]), once per weight."""
    return w8a8_quantize_rows(w)
