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


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(q[45]k_\w+)\(", text, re.M)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for name in ("q4k_gemv", "q4k_gemm", "q4k_swiglu_mlp", "q4k_init", "q4k_last_error",
                 "q4k_dequantize_f32", "q4k_dequantize_bf16", "q4k_device_name", "q4k_version",
                 "q5k_gemv", "q5k_gemm", "q5k_dequantize_f32", "q5k_dequantize_bf16"):
        assert name in syms


def test_library_loads_and_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert set(declared_symbols()) == set(_lib.SIGNATURES)
    assert _lib.q4k_version() >= 100


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ("Q4K_OK", "Q4K_ERR_INVALID_ARG", "Q4K_ERR_ALIGN", "Q4K_ERR_DEVICE",
                 "Q4K_ERR_LAUNCH", "Q4K_QK", "Q4K_BLOCK_BYTES", "Q4K_GEMV_MAX_M",
                 "Q5K_BLOCK_BYTES"):
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
