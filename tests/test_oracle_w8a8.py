"""Pins of the INT8 W8A8 oracle to facts fixed outside it.

The oracle (``oracle/w8a8_oracle.c``) follows the INT8 linear layer of the
xpu-kernels page ("API", "Use from C"): an exact int8 x int8 -> int32
contraction, the epilogue acc * x_scale[m] * w_scale[n] + bias[n] to bf16, and
a per-row absmax quantizer.  Each test below checks it against something it
does not compute itself: pure-Python integer sums, numpy's int64 matmul,
closed forms, and hand-derived IEEE roundings.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth


def _f32_bits(v: float) -> int:
    return int(np.array([v], np.float32).view(np.uint32)[0])


def _bf16_value(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- accumulator

def test_acc_matches_python_integer_sums():
    # int8 extremes (-128 included), k not a multiple of anything
    x = synth.int8_uniform((3, 37), seed=11, stream=synth.X)
    w = synth.int8_uniform((4, 37), seed=11, stream=synth.W)
    acc = oracle.w8a8_acc(x, w)
    for i in range(3):
        for j in range(4):
            assert acc[i, j] == sum(int(x[i, c]) * int(w[j, c]) for c in range(37))


def test_acc_matches_numpy_int64_matmul():
    x = synth.int8_codes((17, 1000), seed=12, stream=synth.X)
    w = synth.int8_codes((33, 1000), seed=12, stream=synth.W)
    ref = x.astype(np.int64) @ w.astype(np.int64).T
    np.testing.assert_array_equal(oracle.w8a8_acc(x, w), ref)


def test_acc_closed_forms():
    w = synth.int8_uniform((5, 300), seed=13, stream=synth.W)
    # all-ones activation row: the weight row sums
    ones = np.ones((1, 300), np.int8)
    np.testing.assert_array_equal(oracle.w8a8_acc(ones, w)[0], w.astype(np.int64).sum(1))
    # one-hot activation rows pick weight columns
    eye = np.zeros((3, 300), np.int8)
    for i, c in enumerate((0, 151, 299)):
        eye[i, c] = 1
    acc = oracle.w8a8_acc(eye, w)
    for i, c in enumerate((0, 151, 299)):
        np.testing.assert_array_equal(acc[i], w[:, c].astype(np.int64))
    # extremes: (-128)(-128) k and 127 (-128) k
    k = 3072
    lo = np.full((1, k), -128, np.int8)
    hi = np.full((1, k), 127, np.int8)
    assert oracle.w8a8_acc(lo, lo)[0, 0] == 16384 * k
    assert oracle.w8a8_acc(hi, lo)[0, 0] == -16256 * k


def test_acc_rejects_int32_overflow():
    k = 131072  # 16384 * 131072 = 2^31, one past INT32_MAX
    lo = np.full((1, k), -128, np.int8)
    with pytest.raises(ValueError):
        oracle.w8a8_acc(lo, lo)
    ok = np.full((1, k - 1), -128, np.int8)
    assert oracle.w8a8_acc(ok, ok)[0, 0] == 16384 * (k - 1)


# ------------------------------------------------------------------- epilogue

def _epi(acc, xs, ws, bias):
    acc = np.array([[acc]], np.int32)
    b = None if bias is None else np.array([bias], np.float32)
    out, f = oracle.w8a8_epilogue(acc, np.array([xs], np.float32), np.array([ws], np.float32), b)
    return int(out[0, 0]), float(f[0, 0])


def test_epilogue_hand_values():
    # 3 * 0.5 * 0.25 + 1 = 1.375 exactly; bf16 0x3FB0
    assert _epi(3, 0.5, 0.25, 1.0) == (0x3FB0, 1.375)
    # no bias: 3 * 0.5 * 0.25 = 0.375; bf16 0x3EC0
    assert _epi(3, 0.5, 0.25, None) == (0x3EC0, 0.375)
    # negative accumulator and bias
    assert _epi(-40, 0.25, 0.5, -1.0) == (0xC0C0, -6.0)


def test_epilogue_bf16_ties_go_to_even():
    # 1 + 2^-8 lies halfway between bf16 1.0 (even) and 1 + 2^-7 (odd)
    assert _epi(1, 1.0, 1.0, 2.0 ** -8) == (0x3F80, 1.0 + 2.0 ** -8)
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert _epi(1, 1.0, 1.0, 3 * 2.0 ** -8) == (0x3F82, 1.0 + 3 * 2.0 ** -8)
    # just above the first tie rounds up
    assert _epi(1, 1.0, 1.0, 2.0 ** -8 + 2.0 ** -20)[0] == 0x3F81


def test_epilogue_converts_the_accumulator_to_nearest_even_fp32():
    # 2^24 + 1 is a tie between 2^24 (even) and 2^24 + 2; 2^24 + 3 between 2^24 + 2 and + 4 (even)
    assert _epi(2 ** 24 + 1, 1.0, 1.0, None)[1] == 2.0 ** 24
    assert _epi(2 ** 24 + 3, 1.0, 1.0, None)[1] == 2.0 ** 24 + 4
    assert _epi(-(2 ** 24 + 3), 1.0, 1.0, None)[1] == -(2.0 ** 24 + 4)


def test_epilogue_rounds_every_operation_left_to_right():
    # Unfused multiply-add: (1 + 2^-12)^2 = 1 + 2^-11 + 2^-24 rounds to 1 + 2^-11 (a tie,
    # to even); minus 1 gives 2^-11.  A fused multiply-add would keep the 2^-24.
    e = 1.0 + 2.0 ** -12
    assert _epi(1, e, e, -1.0)[1] == 2.0 ** -11
    # Left to right: 3 (1 + 2^-23) = 3 + 1.5 ulp(3) rounds to 3 + 2^-21 (even); times
    # (1 + 2^-23) gives 3 + 3.5 * 2^-22 + 2^-44, rounding to 3 + 2^-20.  Multiplying the
    # scales first would give 3 (1 + 2^-22) = 3 + 3 * 2^-22 exactly.
    u = 1.0 + 2.0 ** -23
    assert _epi(3, u, u, None)[1] == 3.0 + 2.0 ** -20


def test_epilogue_scales_exactly_by_powers_of_two():
    x, xs, w, ws, _ = synth.w8a8_case(6, 9, 512, seed=14)
    acc = oracle.w8a8_acc(x, w)
    _, f1 = oracle.w8a8_epilogue(acc, xs, ws)
    _, f2 = oracle.w8a8_epilogue(acc, xs * 4, ws)
    np.testing.assert_array_equal(f2, f1 * 4)
    out1, _ = oracle.w8a8_epilogue(-acc, xs, ws)
    np.testing.assert_array_equal(_bf16_value(out1), -_bf16_value(oracle.w8a8_epilogue(acc, xs, ws)[0]))


def test_epilogue_is_close_to_the_exact_product():
    # |bf16 - exact| <= 2^-8 |exact| (bf16 rounding) + a few fp32 roundings
    x, xs, w, ws, b = synth.w8a8_case(8, 12, 1024, seed=15)
    acc = oracle.w8a8_acc(x, w)
    out, _ = oracle.w8a8_epilogue(acc, xs, ws, b)
    exact = acc.astype(np.float64) * xs.astype(np.float64)[:, None] * ws.astype(np.float64)[None, :] \
        + b.astype(np.float64)[None, :]
    got = _bf16_value(out).astype(np.float64)
    assert np.all(np.abs(got - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-6 * (np.abs(exact) + np.abs(b)))


def test_linear_and_sampled_columns_agree_with_acc_then_epilogue():
    x, xs, w, ws, b = synth.w8a8_case(5, 40, 768, seed=16)
    acc = oracle.w8a8_acc(x, w)
    out, _ = oracle.w8a8_epilogue(acc, xs, ws, b)
    np.testing.assert_array_equal(oracle.w8a8_linear(x, xs, w, ws, b), out)
    cols = np.array([0, 7, 39, 20])
    np.testing.assert_array_equal(oracle.w8a8_linear_cols(x, xs, w, ws, b, cols), out[:, cols])
    out_nb, _ = oracle.w8a8_epilogue(acc, xs, ws)
    np.testing.assert_array_equal(oracle.w8a8_linear(x, xs, w, ws, None), out_nb)


# ------------------------------------------------------------------ quantizer

def _bits(values) -> np.ndarray:
    return synth.bf16_bits(np.asarray(values, np.float32).reshape(1, -1))


def test_quantizer_hand_row_with_unit_scale():
    # amax = 127 gives scale 1 exactly, so the codes are the values rounded half to even
    row = [127.0, 1.0, -64.0, 0.5, 63.5, 62.5, -0.5, -1.5, 2.5, -127.0]
    q, s = oracle.w8a8_quantize_rows(_bits(row))
    assert s[0] == 1.0
    assert q[0].tolist() == [127, 1, -64, 0, 64, 62, 0, -2, 2, -127]


def test_quantizer_zero_row():
    q, s = oracle.w8a8_quantize_rows(np.zeros((2, 64), np.uint16))
    assert s.tolist() == [0.0, 0.0] and not q.any()


def test_quantizer_properties():
    xb = synth.normal_bf16((16, 3072), seed=17)
    q, s = oracle.w8a8_quantize_rows(xb)
    x = _bf16_value(xb).astype(np.float64)
    amax = np.abs(x).max(1)
    # scale = amax / 127 rounded to fp32
    np.testing.assert_array_equal(s, (amax / 127).astype(np.float32))
    # codes in range and the row maximum maps to +-127
    assert np.abs(q.astype(int)).max() <= 127
    np.testing.assert_array_equal(np.abs(q.astype(int)).max(1), 127)
    # rounding error at most half a step (plus the fp32 division's own error)
    err = np.abs(q.astype(np.float64) * s[:, None] - x)
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 2.0 ** -17))
    # odd symmetry and exact power-of-two scaling
    q_neg, s_neg = oracle.w8a8_quantize_rows(xb ^ np.uint16(0x8000))
    np.testing.assert_array_equal(q_neg, -q)
    np.testing.assert_array_equal(s_neg, s)
    q2, s2 = oracle.w8a8_quantize_rows(synth.bf16_bits((x * 8).astype(np.float32)))
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(s2, s * 8)


def test_quantizer_tiny_row():
    q, s = oracle.w8a8_quantize_rows(_bits([1e-30, -2e-30, 0.0]))
    assert s[0] > 0 and q[0].tolist()[1] == -127 and q[0].tolist()[2] == 0
