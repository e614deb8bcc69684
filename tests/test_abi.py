"""The C ABI without a GPU: symbols, argument validation, shipped shapes.

No test here launches a kernel: every call either fails host-side validation
(which runs before anything touches the device) or, on a machine without a
GPU, stops at the device check.
"""
from __future__ import annotations

import os
import re

import pytest

import torch

from gemm_q4_super_block_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4k.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


def declared_symbols():
    text = "\n".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?((?:q[3456]k|w8a8)_\w+)\(",
                                 text, re.M)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for name in ("q4k_gemv", "q4k_gemm", "q4k_swiglu_mlp", "q4k_init", "q4k_last_error",
                 "q4k_dequantize_f32", "q4k_dequantize_bf16", "q4k_device_name", "q4k_version",
                 "q5k_gemv", "q5k_gemm", "q5k_dequantize_f32", "q5k_dequantize_bf16",
                 "q6k_gemv", "q6k_dequantize_f32", "q6k_dequantize_bf16", "q3k_gemv",
                 "q3k_dequantize_f32", "q3k_dequantize_bf16", "q6k_gemm", "q3k_gemm",
                 "w8a8_linear", "w8a8_linear_acc", "w8a8_dequant_epilogue", "w8a8_quantize_rows"):
        assert name in syms


def test_library_loads_and_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert set(declared_symbols()) == set(_lib.SIGNATURES)
    assert _lib.q4k_version() >= 100


def test_header_constants_match_binding():
    text = "\n".join(open(h).read() for h in HEADERS)
    for name in ("Q4K_OK", "Q4K_ERR_INVALID_ARG", "Q4K_ERR_ALIGN", "Q4K_ERR_DEVICE",
                 "Q4K_ERR_LAUNCH", "Q4K_QK", "Q4K_BLOCK_BYTES", "Q4K_GEMV_MAX_M",
                 "Q5K_BLOCK_BYTES", "Q6K_BLOCK_BYTES", "Q3K_BLOCK_BYTES", "W8A8_K_STEP",
                 "W8A8_MAX_K", "Q4K_MAX_N", "Q4K_GEMM_MAX_K", "Q4K_NOALLOC_MAX_D_FF",
                 "Q4K_LAYERS_MAX", "Q4K_LAYERS_MAX_K"):
        mm = re.search(r"#define %s \(?(-?\d+)\)?" % name, text)
        assert mm, name
        assert int(mm.group(1)) == getattr(_lib, name), name


A = 1 << 20  # a 16-byte-aligned fake address: never dereferenced (validation fails first)


@pytest.mark.parametrize("args,code", [
    ((0, A, 2 * A, 1, 16, 256), _lib.Q4K_ERR_INVALID_ARG),        # null w
    ((A, 0, 2 * A, 1, 16, 256), _lib.Q4K_ERR_INVALID_ARG),        # null x
    ((A, 2 * A, 0, 1, 16, 256), _lib.Q4K_ERR_INVALID_ARG),        # null y
    ((A, 2 * A, 3 * A, 0, 16, 256), _lib.Q4K_ERR_INVALID_ARG),    # m = 0
    ((A, 2 * A, 3 * A, 33, 16, 256), _lib.Q4K_ERR_INVALID_ARG),   # m > 32
    ((A, 2 * A, 3 * A, 1, 0, 256), _lib.Q4K_ERR_INVALID_ARG),     # n = 0
    ((A, 2 * A, 3 * A, 1, 16, 300), _lib.Q4K_ERR_INVALID_ARG),    # k % 256
    ((A, 2 * A, 3 * A, 1, 16, 0), _lib.Q4K_ERR_INVALID_ARG),      # k = 0
    ((A, 2 * A, 3 * A, 1, 16, -256), _lib.Q4K_ERR_INVALID_ARG),   # k < 0
    ((A + 4, 2 * A, 3 * A, 1, 16, 256), _lib.Q4K_ERR_ALIGN),      # misaligned w
    ((A, 2 * A + 8, 3 * A, 1, 16, 256), _lib.Q4K_ERR_ALIGN),      # misaligned x
    ((A, 2 * A, 2 * A + 16, 1, 16, 256), _lib.Q4K_ERR_INVALID_ARG),  # y overlaps x
])
def test_gemv_rejects_bad_arguments(args, code):
    assert _lib.q4k_gemv(*args, None) == code
    assert _lib.q4k_last_error().startswith("q4k_gemv")


@pytest.mark.parametrize("args,code", [
    ((0, A, 2 * A, 8, 16, 256), _lib.Q4K_ERR_INVALID_ARG),
    ((A, 2 * A, 3 * A, 0, 16, 256), _lib.Q4K_ERR_INVALID_ARG),
    ((A, 2 * A, 3 * A, 8, 16, 512 + 128), _lib.Q4K_ERR_INVALID_ARG),
    ((A, 2 * A + 2, 3 * A, 8, 16, 256), _lib.Q4K_ERR_ALIGN),
    ((A, 2 * A, A + 16, 8, 16, 256), _lib.Q4K_ERR_INVALID_ARG),   # y overlaps w
])
def test_gemm_rejects_bad_arguments(args, code):
    assert _lib.q4k_gemm(*args, None) == code


def test_mlp_rejects_bad_arguments():
    good = (A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, 256, 512)
    bad_null = (A, 0) + good[2:]
    assert _lib.q4k_swiglu_mlp(*bad_null, None) == _lib.Q4K_ERR_INVALID_ARG
    bad_k = good[:6] + (256, 500)
    assert _lib.q4k_swiglu_mlp(*bad_k, None) == _lib.Q4K_ERR_INVALID_ARG
    bad_align = good[:4] + (5 * A + 4, 6 * A, 256, 512)
    assert _lib.q4k_swiglu_mlp(*bad_align, None) == _lib.Q4K_ERR_ALIGN
    alias = good[:4] + (4 * A, 6 * A, 256, 512)  # h == x
    assert _lib.q4k_swiglu_mlp(*alias, None) == _lib.Q4K_ERR_INVALID_ARG


def test_dequant_rejects_bad_arguments():
    assert _lib.q4k_dequantize_f32(0, A, 4, 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q4k_dequantize_bf16(A, 2 * A, 4, 100, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q4k_dequantize_f32(A, 2 * A + 4, 4, 256, None) == _lib.Q4K_ERR_ALIGN


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is present")
def test_no_device_is_reported_cleanly():
    assert _lib.q4k_init() == _lib.Q4K_ERR_DEVICE
    assert "device" in _lib.q4k_last_error()
    assert _lib.q4k_device_name() == "none"
    # valid-looking arguments stop at the device check, before any launch
    assert _lib.q4k_gemv(A, 2 * A, 3 * A, 1, 16, 256, None) == _lib.Q4K_ERR_DEVICE


def test_shipped_launch_shapes_are_pinned():
    src = os.path.join(ROOT, "gemm_q4_super_block_amd", "csrc")
    launch = open(os.path.join(src, "q4k_launch.h")).read()
    assert re.search(r"kGemvRowsPerWave = 1;", launch)
    assert re.search(r"kGemvWideRows = 8192;", launch)
    assert re.search(r"kDecodeWaves = 8;", launch)
    assert re.search(r"kGateUpRowsPerWave = 1;", launch)
    gemm = open(os.path.join(src, "k_gemm.hip")).read()
    assert re.search(r"kBN = 128;", gemm) and re.search(r"kBK = 64;", gemm)


def test_ops_reject_cpu_tensors():
    import gemm_q4_super_block_amd as q4k
    w = torch.zeros((4, 144), dtype=torch.uint8)
    with pytest.raises(ValueError):
        q4k.gemv(w, torch.zeros(256))


def test_read_probe_rejects_bad_arguments():
    assert _lib.q4k_read_probe(0, 4096, A, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q4k_read_probe(A, 0, 2 * A, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q4k_read_probe(A, 4100, 2 * A, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q4k_read_probe(A + 4, 4096, 2 * A, None) == _lib.Q4K_ERR_ALIGN
    assert _lib.q4k_read_probe(A, 4096, 2 * A + 2, None) == _lib.Q4K_ERR_ALIGN
    assert _lib.q4k_read_probe(A, 4096, A + 64, None) == _lib.Q4K_ERR_INVALID_ARG  # sink in buf
    assert _lib.q4k_last_error().startswith("q4k_read_probe")


def test_q5k_rejects_bad_arguments():
    assert _lib.q5k_gemv(0, A, 2 * A, 1, 16, 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q4k_last_error().startswith("q5k_gemv")
    assert _lib.q5k_gemv(A, 2 * A, 3 * A, 33, 16, 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q5k_gemv(A, 2 * A, 3 * A, 1, 16, 300, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q5k_gemv(A + 8, 2 * A, 3 * A, 1, 16, 256, None) == _lib.Q4K_ERR_ALIGN
    # 16 rows of one 176-byte block span 2816 bytes from A: y may not start inside
    assert _lib.q5k_gemv(A, 2 * A, A + 2800, 1, 16, 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q5k_gemm(A, 2 * A, 3 * A, 8, 16, 300, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q5k_gemm(A, 2 * A + 2, 3 * A, 8, 16, 256, None) == _lib.Q4K_ERR_ALIGN
    assert _lib.q5k_gemm(A, 2 * A, A + 2800, 8, 16, 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q4k_last_error().startswith("q5k_gemm")
    assert _lib.q5k_dequantize_f32(0, A, 4, 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q5k_dequantize_bf16(A, 2 * A + 4, 4, 256, None) == _lib.Q4K_ERR_ALIGN
    assert _lib.q5k_dequantize_f32(A, A + 688, 4, 256, None) == _lib.Q4K_ERR_INVALID_ARG  # out in w
    assert _lib.q4k_last_error().startswith("q5k_dequantize_f32")


def test_w8a8_max_k_keeps_every_sum_in_int32():
    assert _lib.W8A8_MAX_K % _lib.W8A8_K_STEP == 0
    assert 128 * 128 * _lib.W8A8_MAX_K <= 2 ** 31 - 1
    assert 128 * 128 * (_lib.W8A8_MAX_K + _lib.W8A8_K_STEP) > 2 ** 31 - 1


def test_w8a8_rejects_bad_arguments():
    lin = _lib.w8a8_linear
    X, XS, W, WS, B, O = A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A
    E = _lib.Q4K_ERR_INVALID_ARG
    assert lin(0, XS, W, WS, B, O, 4, 8, 128, None) == E                  # null x
    assert _lib.q4k_last_error().startswith("w8a8_linear")
    assert lin(X, 0, W, WS, B, O, 4, 8, 128, None) == E                   # null x_scale
    assert lin(X, XS, W, WS, B, 0, 4, 8, 128, None) == E                  # null out
    assert lin(X, XS, W, WS, B, O, 0, 8, 128, None) == E                  # m = 0
    assert lin(X, XS, W, WS, B, O, 4, 0, 128, None) == E                  # n = 0
    assert lin(X, XS, W, WS, B, O, 4, 8, 64, None) == E                   # k % 128
    assert lin(X, XS, W, WS, B, O, 4, 8, 0, None) == E                    # k = 0
    assert lin(X, XS, W, WS, B, O, 4, 8, _lib.W8A8_MAX_K + 128, None) == E  # sums overflow
    assert lin(X + 8, XS, W, WS, B, O, 4, 8, 128, None) == _lib.Q4K_ERR_ALIGN
    assert lin(X, XS, W, WS, B, O + 2, 4, 8, 128, None) == _lib.Q4K_ERR_ALIGN
    assert lin(X, XS + 2, W, WS, B, O, 4, 8, 128, None) == _lib.Q4K_ERR_ALIGN
    assert lin(X, XS, W, WS, B, X + 256, 4, 8, 128, None) == E            # out inside x
    assert lin(X, XS, W, WS, O + 32, O, 4, 8, 128, None) == E             # bias inside out
    acc = _lib.w8a8_linear_acc
    assert acc(X, W, 0, 4, 8, 128, None) == E
    assert acc(X, W, O, 4, 8, 100, None) == E
    assert acc(X, W + 4, O, 4, 8, 128, None) == _lib.Q4K_ERR_ALIGN
    assert acc(X, W, W + 16, 4, 8, 128, None) == E                        # acc inside w
    assert _lib.q4k_last_error().startswith("w8a8_linear_acc")
    epi = _lib.w8a8_dequant_epilogue
    assert epi(0, O, XS, WS, B, 4, 8, None) == E
    assert epi(X, O, 0, WS, B, 4, 8, None) == E
    assert epi(X, O, XS, WS, B, 0, 8, None) == E
    assert epi(X + 4, O, XS, WS, B, 4, 8, None) == _lib.Q4K_ERR_ALIGN
    assert epi(X, X + 64, XS, WS, B, 4, 8, None) == E                     # out inside acc
    assert _lib.q4k_last_error().startswith("w8a8_dequant_epilogue")
    qr = _lib.w8a8_quantize_rows
    assert qr(0, O, XS, 4, 128, None) == E
    assert qr(X, O, XS, 4, 12, None) == E                                 # k % 8
    assert qr(X, O, XS, 0, 128, None) == E
    assert qr(X, O + 8, XS, 4, 128, None) == _lib.Q4K_ERR_ALIGN
    assert qr(X, X + 512, XS, 4, 128, None) == E                          # q inside x
    assert _lib.q4k_last_error().startswith("w8a8_quantize_rows")


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is present")
def test_w8a8_valid_arguments_stop_at_the_device_check():
    assert _lib.w8a8_linear(A, 2 * A, 3 * A, 4 * A, 0, 6 * A, 4, 8, 128, None) == _lib.Q4K_ERR_DEVICE
    assert _lib.w8a8_quantize_rows(A, 2 * A, 3 * A, 4, 128, None) == _lib.Q4K_ERR_DEVICE


def test_q6k_rejects_bad_arguments():
    assert _lib.q6k_gemv(0, A, 2 * A, 1, 16, 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q4k_last_error().startswith("q6k_gemv")
    assert _lib.q6k_gemv(A, 2 * A, 3 * A, 33, 16, 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q6k_gemv(A, 2 * A, 3 * A, 1, 16, 200, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q6k_gemv(A + 2, 2 * A, 3 * A, 1, 16, 256, None) == _lib.Q4K_ERR_ALIGN
    # 16 rows of one 210-byte block span 3360 bytes from A: y may not start inside
    assert _lib.q6k_gemv(A, 2 * A, A + 3344, 1, 16, 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q6k_dequantize_f32(0, A, 4, 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q6k_dequantize_bf16(A, 2 * A + 4, 4, 256, None) == _lib.Q4K_ERR_ALIGN
    assert _lib.q6k_dequantize_f32(A, A + 832, 4, 256, None) == _lib.Q4K_ERR_INVALID_ARG  # out in w
    assert _lib.q4k_last_error().startswith("q6k_dequantize_f32")


def test_q3k_rejects_bad_arguments():
    assert _lib.q3k_gemv(0, A, 2 * A, 1, 16, 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q4k_last_error().startswith("q3k_gemv")
    assert _lib.q3k_gemv(A, 2 * A, 3 * A, 33, 16, 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q3k_gemv(A, 2 * A, 3 * A, 1, 16, 384, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q3k_gemv(A + 4, 2 * A, 3 * A, 1, 16, 256, None) == _lib.Q4K_ERR_ALIGN
    # 16 rows of one 110-byte block span 1760 bytes from A: y may not start inside
    assert _lib.q3k_gemv(A, 2 * A, A + 1744, 1, 16, 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q3k_dequantize_bf16(A, 2 * A + 2, 4, 256, None) == _lib.Q4K_ERR_ALIGN
    assert _lib.q3k_dequantize_f32(A, A + 432, 4, 256, None) == _lib.Q4K_ERR_INVALID_ARG  # out in w
    assert _lib.q4k_last_error().startswith("q3k_dequantize_f32")


def test_plane_gemms_reject_bad_arguments():
    for name, blk in (("q6k_gemm", 210), ("q3k_gemm", 110)):
        fn = getattr(_lib, name)
        assert fn(0, A, 2 * A, 8, 16, 256, None) == _lib.Q4K_ERR_INVALID_ARG
        assert _lib.q4k_last_error().startswith(name)
        assert fn(A, 2 * A, 3 * A, 8, 16, 300, None) == _lib.Q4K_ERR_INVALID_ARG
        assert fn(A + 2, 2 * A, 3 * A, 8, 16, 256, None) == _lib.Q4K_ERR_ALIGN
        assert fn(A, 2 * A, A + 16 * blk - 16, 8, 16, 256, None) == _lib.Q4K_ERR_INVALID_ARG  # y in w


def test_gemms_reject_k_past_the_stated_limit():
    # A 256-row weight tile must span < 4 GiB (in-tile offsets are 32-bit, the
    # tile base 64-bit): k above Q4K_GEMM_MAX_K is refused for every format.
    big_k = _lib.Q4K_GEMM_MAX_K + 256
    for name in ("q4k_gemm", "q5k_gemm", "q6k_gemm", "q3k_gemm"):
        fn = getattr(_lib, name)
        assert fn(A, 2 * A, 3 * A, 8, 16, big_k, None) == _lib.Q4K_ERR_INVALID_ARG, name
        assert "Q4K_GEMM_MAX_K" in _lib.q4k_last_error()
    assert 256 * (_lib.Q4K_GEMM_MAX_K // 256) * 176 < 2 ** 32  # largest record, Q5_K


def test_n_past_the_stated_limit_is_rejected():
    n = _lib.Q4K_MAX_N + 1
    assert _lib.q4k_gemv(A, 2 * A, 3 * A, 1, n, 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.q4k_gemm(A, 2 * A, 3 * A, 8, n, 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert _lib.Q4K_MAX_N + 65536 == 2 ** 31 - 1


def test_gemm_weight_offsets_are_tile_relative():
    # The LDS-copy GEMM kernels form each weight row's byte offset from a
    # 64-bit tile base, never as a 32-bit row * row_bytes over the whole matrix.
    src = open(os.path.join(ROOT, "gemm_q4_super_block_amd", "csrc", "k_gemm.hip")).read()
    assert "static_cast<uint32_t>(min(n0 + col" not in src
    assert src.count("w + static_cast<size_t>(n0) * row_bytes") == 2


class _FakeTensor:
    """Stands in for a CUDA tensor so the binding's output checks run on the CPU."""

    def __init__(self, shape, dtype=torch.float32, device="cuda:0"):
        self.shape = torch.Size(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self.is_cuda = True

    def is_contiguous(self):
        return True


def test_binding_output_checks():
    from gemm_q4_super_block_amd import ops
    dev = torch.device("cuda:0")
    ops._out_tensor(_FakeTensor((3, 64)), torch.float32, (3, 64), dev, "out")
    for bad in (_FakeTensor((3, 63)), _FakeTensor((192,)), _FakeTensor((3, 64), torch.float64),
                _FakeTensor((3, 64), device="cuda:1")):
        with pytest.raises(ValueError):
            ops._out_tensor(bad, torch.float32, (3, 64), dev, "out")


def test_noalloc_mlp_rejects_bad_arguments():
    fn = _lib.q4k_swiglu_mlp_noalloc
    good = (A, 2 * A, 3 * A, 4 * A, 5 * A, 256, 512)
    assert fn(0, *good[1:], None) == _lib.Q4K_ERR_INVALID_ARG
    assert fn(*good[:5], 256, _lib.Q4K_NOALLOC_MAX_D_FF + 256, None) == _lib.Q4K_ERR_INVALID_ARG
    assert "Q4K_NOALLOC_MAX_D_FF" in _lib.q4k_last_error()
    assert fn(*good[:4], 5 * A + 4, 256, 512, None) == _lib.Q4K_ERR_ALIGN
    assert fn(*good[:4], 4 * A, 256, 512, None) == _lib.Q4K_ERR_INVALID_ARG  # out == x


def test_gemv_layers_rejects_bad_arguments():
    f = _lib.q4k_gemv_layers
    W = [A, A + (1 << 16)]
    X = [2 * A, 2 * A + 4096]
    Y = [3 * A, 3 * A + 4096]
    E = _lib.Q4K_ERR_INVALID_ARG
    assert f([], [], [], 16, 256, None) == E                              # no layers
    assert "layers" in _lib.q4k_last_error()
    assert f([A] * 33, [2 * A] * 33, [3 * A + 256 * i for i in range(33)], 16, 256, None) == E
    assert f([A, 0], X, Y, 16, 256, None) == E                            # null w[1]
    assert f(W, X, Y, 16, 300, None) == E                                 # k % 256
    assert f(W, X, Y, 16, _lib.Q4K_LAYERS_MAX_K + 256, None) == E         # k past the limit
    assert f(W, [2 * A, 2 * A + 8], Y, 16, 256, None) == _lib.Q4K_ERR_ALIGN
    assert f(W, X, [3 * A, 3 * A + 32], 16, 256, None) == E               # y[0] and y[1] overlap
    assert f(W, X, [3 * A, 2 * A + 4096], 16, 256, None) == E             # y[1] is x[1]
    assert f(W, X, [3 * A, W[0] + 64], 16, 256, None) == E                # y[1] inside w[0]
    assert _lib.q4k_last_error().startswith("q4k_gemv_layers")
