"""Parity of the INT8 W8A8 entry points with the oracle, bit for bit.

Integer accumulation is exact and the epilogue is a fixed sequence of fp32
operations, each rounded on its own, so every output is compared bit for bit:
int32 accumulators, bf16 outputs, int8 codes and fp32 scales.  Shapes: the
pages' workload (K = N = 3072, M from 512 to 8192) at full size on sampled
columns, smaller cases in full with ragged M and N tiles, a single output,
the largest K, and the extremes of int8.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4k():
    if torch.cuda.device_count() == 0:
        pytest.skip("no GPU")
    import gemm_q4_super_block_amd as lib
    lib.load_library()
    torch.cuda.set_device(0)
    return lib


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_bits(got: np.ndarray, ref: np.ndarray, what: str):
    bad = got != ref
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError("%s: %d of %d outputs differ, first at %s" % (what, bad.sum(), bad.size,
                                                                          idx))


def run_linear(q4k, case, bias=True):
    x, xs, w, ws, b = case
    return bits16(q4k.w8a8_linear(dev(x), dev(xs), dev(w), dev(ws), dev(b) if bias else None))


@pytest.mark.parametrize("m,n,k,seed", [
    (128, 128, 128, 0),     # one tile, one K step
    (256, 384, 1024, 1),    # several tiles, eight steps
    (130, 200, 384, 2),     # ragged M and N tiles
    (1, 1, 256, 3),         # a single output
    (64, 1024, 512, 4),     # one row of 64 x 64 tiles (small grids)
    (257, 129, 640, 5),     # ragged, odd step count
    (96, 3072, 3072, 6),    # the pages' K and N, small M
    (2100, 2000, 256, 7),   # 128 x 128 tiles (more than 256 of them), ragged
    (1030, 3072, 256, 8),   # 64 x 192 tiles, three-slot ring (a small grid that fills the CUs), ragged M
    (2200, 1900, 256, 9),   # 128 x 192 tiles (a large grid), ragged M and N
])
def test_linear_acc_and_fused_epilogue_bit_exact(q4k, m, n, k, seed):
    case = synth.w8a8_case(m, n, k, seed)
    x, xs, w, ws, b = case
    acc = q4k.w8a8_linear_acc(dev(x), dev(w)).cpu().numpy()
    assert_bits(acc, oracle.w8a8_acc(x, w), "acc %dx%dx%d" % (m, n, k))
    assert_bits(run_linear(q4k, case), oracle.w8a8_linear(x, xs, w, ws, b), "linear")
    assert_bits(run_linear(q4k, case, bias=False), oracle.w8a8_linear(x, xs, w, ws, None),
                "linear without bias")


@pytest.mark.parametrize("m", [512, 1024, 8192])
def test_linear_full_size_sampled_columns(q4k, m):
    n = k = 3072
    case = synth.w8a8_case(m, n, k, seed=7)
    x, xs, w, ws, b = case
    got = run_linear(q4k, case)
    cols = np.array([0, 1, 127, 128, 1000, 1535, 2047, 2048, 2500, 3071])
    assert_bits(got[:, cols], oracle.w8a8_linear_cols(x, xs, w, ws, b, cols),
                "linear m=%d sampled columns" % m)


def test_fused_equals_acc_then_dequant(q4k):
    # the page's claim: dequant(linear_acc(...)) is bit-identical to linear(...)
    x, xs, w, ws, b = synth.w8a8_case(1024, 3072, 3072, seed=8)
    X, XS, W, WS, B = dev(x), dev(xs), dev(w), dev(ws), dev(b)
    fused = bits16(q4k.w8a8_linear(X, XS, W, WS, B))
    two = bits16(q4k.w8a8_dequant(q4k.w8a8_linear_acc(X, W), XS, WS, B))
    assert_bits(fused, two, "fused vs acc + epilogue")


@pytest.mark.parametrize("m,n,bias", [(64, 3072, True), (5, 7, True), (33, 130, False),
                                      (1, 1, True)])
def test_standalone_epilogue_bit_exact(q4k, m, n, bias):
    g = synth.rng(9, 0)
    acc = g.integers(-2 ** 31, 2 ** 31, size=(m, n), dtype=np.int64).astype(np.int32)
    xs = synth.uniform_f32((m,), 0.01, 0.05, seed=9)
    ws = synth.uniform_f32((n,), 2e-4, 1e-3, seed=9, stream=synth.W_SCALE)
    b = synth.uniform_f32((n,), -1.0, 1.0, seed=9, stream=synth.BIAS) if bias else None
    got = bits16(q4k.w8a8_dequant(dev(acc), dev(xs), dev(ws), None if b is None else dev(b)))
    assert_bits(got, oracle.w8a8_epilogue(acc, xs, ws, b)[0], "epilogue %dx%d" % (m, n))


def test_epilogue_rounding_cases(q4k):
    # inputs that hit the oracle's hand-derived cases: bf16 ties (row 0, columns 0 and 1), an
    # int32 -> fp32 tie (row 0, column 2), a product whose fused multiply-add would differ
    # (row 1, column 3) and a result that depends on the order of the two scalings (row 2,
    # column 4)
    e = 1.0 + 2.0 ** -12
    u = 1.0 + 2.0 ** -23
    acc = np.array([[1, 1, 2 ** 24 + 3, 5, 7], [2, 3, 4, 1, 6], [1, 2, 3, 4, 3]], np.int32)
    xs = np.array([1.0, e, u], np.float32)
    ws = np.array([1.0, 1.0, 1.0, e, u], np.float32)
    b = np.array([2.0 ** -8, 3 * 2.0 ** -8, 0.0, -1.0, 0.0], np.float32)
    got = bits16(q4k.w8a8_dequant(dev(acc), dev(xs), dev(ws), dev(b)))
    ref, ref_f32 = oracle.w8a8_epilogue(acc, xs, ws, b)
    assert ref_f32[1, 3] == 2.0 ** -11 and ref_f32[2, 4] == 3.0 + 2.0 ** -20
    assert_bits(got, ref, "rounding cases")


def test_int8_extremes_and_largest_k(q4k):
    k = 130944  # the largest accepted k: 128 * 128 * k still fits in int32
    lo = np.full((2, k), -128, np.int8)
    acc = q4k.w8a8_linear_acc(dev(lo), dev(lo)).cpu().numpy()
    assert (acc == 16384 * k).all()
    hi = np.full((1, k), 127, np.int8)
    acc = q4k.w8a8_linear_acc(dev(hi), dev(lo[:1])).cpu().numpy()
    assert (acc == -16256 * k).all()
    x = synth.int8_uniform((70, 4096), seed=10, stream=synth.X)
    w = synth.int8_uniform((150, 4096), seed=10, stream=synth.W)
    assert_bits(q4k.w8a8_linear_acc(dev(x), dev(w)).cpu().numpy(), oracle.w8a8_acc(x, w),
                "uniform int8 codes")


@pytest.mark.parametrize("rows,k,seed", [(1, 8, 0), (7, 3072, 1), (33, 4104, 2), (1024, 3072, 3),
                                         (3, 14336, 4)])
def test_quantize_rows_bit_exact(q4k, rows, k, seed):
    xb = synth.normal_bf16((rows, k), seed=seed)
    q, s = q4k.w8a8_quantize_rows(dev(xb.view(np.int16)).view(torch.bfloat16))
    rq, rs = oracle.w8a8_quantize_rows(xb)
    assert_bits(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), "scales")
    assert_bits(q.cpu().numpy(), rq, "codes")


def test_quantize_hand_rows(q4k):
    rows = np.zeros((3, 16), np.float32)
    rows[0, :10] = [127.0, 1.0, -64.0, 0.5, 63.5, 62.5, -0.5, -1.5, 2.5, -127.0]
    rows[2, :3] = [1e-30, -2e-30, 0.0]  # row 1 stays zero
    xb = synth.bf16_bits(rows)
    q, s = q4k.w8a8_quantize_rows(dev(xb.view(np.int16)).view(torch.bfloat16))
    rq, rs = oracle.w8a8_quantize_rows(xb)
    assert_bits(s.cpu().numpy().view(np.uint32), rs.view(np.uint32), "scales")
    assert_bits(q.cpu().numpy(), rq, "codes")
    assert q.cpu().numpy()[0, :10].tolist() == [127, 1, -64, 0, 64, 62, 0, -2, 2, -127]


def test_quantize_then_linear_end_to_end(q4k):
    # bf16 activations and weights -> codes and scales -> the layer, against the oracle's chain
    m, n, k = 200, 384, 1024
    xb = synth.normal_bf16((m, k), seed=11)
    wb = synth.bf16_bits(synth.normal_f32((n, k), seed=11, stream=synth.W) * 0.02)
    b = synth.uniform_f32((n,), -0.1, 0.1, seed=11, stream=synth.BIAS)
    xq, xs = q4k.w8a8_quantize_rows(dev(xb.view(np.int16)).view(torch.bfloat16))
    wq, ws = q4k.prepare_weight(dev(wb.view(np.int16)).view(torch.bfloat16))
    got = bits16(q4k.w8a8_linear(xq, xs, wq, ws, dev(b)))
    rxq, rxs = oracle.w8a8_quantize_rows(xb)
    rwq, rws = oracle.w8a8_quantize_rows(wb)
    assert_bits(got, oracle.w8a8_linear(rxq, rxs, rwq, rws, b), "quantize + linear")
