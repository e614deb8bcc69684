"""Parity of the Q5_K entry points (q5k_gemv, q5k_dequantize_*) with the oracle.

Same bars as Q4_K: dequantized weights bit-exact (fp32, and bf16 = nearest
even of fp32); GEMV within 1e-4 * sum|w x| per output.  Shapes cover each
batch-1 launch shape (up to 8192 rows; taller with k <= 4096, x in
registers; taller past one K step), ragged K steps, the batched passes and
the degenerate fields of the format.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from golden_io import hand_blocks
from q5k_pack import pack_q5k_block

pytestmark = pytest.mark.gpu

GEMV_TOL = 1e-4


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


def assert_within(got, ref, scale, tol, what):
    err = np.abs(np.asarray(got, np.float64) - ref)
    bad = err > tol * scale
    assert not bad.any(), "%s: %d outputs outside %g * sum|w x|, worst %g" % (
        what, bad.sum(), tol, (err / np.maximum(tol * scale, 1e-300)).max())


def check_dequant(q4k, w, n, k):
    got = q4k.q5k_dequantize_f32(dev(w)).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oracle.q5k_dequant_f32(w, n, k).view(np.uint32))
    got16 = q4k.q5k_dequantize_bf16(dev(w)).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got16, oracle.q5k_dequant_bf16(w, n, k))


@pytest.mark.parametrize("n,k,seed", [(256, 1024, 0), (256, 1024, 1), (37, 768, 2),
                                      (4096, 4096, 0)])
def test_q5k_dequant_bit_exact(q4k, n, k, seed):
    check_dequant(q4k, synth.q5k_weights(n, k, seed=seed), n, k)


def test_q5k_dequant_hand_blocks(q4k):
    blocks = hand_blocks("hand_blocks_q5k.txt", block_bytes=176)
    w = np.stack([b for b, _ in blocks.values()])
    got = q4k.q5k_dequantize_f32(dev(w)).cpu().numpy()
    for row, (_, expected) in zip(got, blocks.values()):
        assert np.array_equal(row.astype(np.float64), expected)
    check_dequant(q4k, w, w.shape[0], 256)


def test_q5k_dequant_degenerate_fields(q4k):
    rng = np.random.default_rng(5)
    rows = []
    for d_bits, dmin_bits in [(0x0001, 0x0000), (0x03FF, 0x0201), (0x7BFF, 0x7BFF),
                              (0x3C00, 0x0000), (0x0000, 0x3C00)]:
        for q in (np.zeros(256, np.int64), np.full(256, 31), np.full(256, 16),
                  rng.integers(0, 32, 256)):
            sc = rng.integers(0, 64, 8)
            mn = rng.integers(0, 64, 8)
            rows.append(pack_q5k_block(d_bits, dmin_bits, sc, mn, q))
    w = np.stack(rows)
    check_dequant(q4k, w, w.shape[0], 256)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_q5k_gemv_small(q4k, seed):
    n, k = 256, 1024
    w = synth.q5k_weights(n, k, seed=seed)
    x = synth.normal_f32(k, seed=seed)
    y = q4k.q5k_gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.q5k_gemv(w, x, n, k)
    assert_within(y, yr[0], a[0], GEMV_TOL, "q5k gemv 256x1024 seed %d" % seed)


@pytest.mark.parametrize("n,k", [(4096, 4096), (1, 256), (300, 768), (33, 4352), (64, 14336),
                                 (8200, 768), (9001, 4096), (8193, 4352)])
def test_q5k_gemv_shapes(q4k, n, k):
    w = synth.q5k_weights(n, k, seed=n % 97)
    x = synth.normal_f32(k, seed=n % 97)
    y = q4k.q5k_gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.q5k_gemv(w, x, n, k)
    assert_within(y, yr[0], a[0], GEMV_TOL, "q5k gemv %dx%d" % (n, k))


@pytest.mark.parametrize("m", [2, 3, 5, 8, 9, 32])
def test_q5k_gemv_batched(q4k, m):
    n, k = 300, 1024
    w = synth.q5k_weights(n, k, seed=m)
    x = synth.normal_f32((m, k), seed=m)
    y = q4k.q5k_gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.q5k_gemv(w, x, n, k)
    assert_within(y, yr, a, GEMV_TOL, "q5k gemv m=%d" % m)


def test_q5k_gemv_unit_vectors_give_columns(q4k):
    # y(e_c) is column c of the dequantized W (one non-zero product per row):
    # exactly on the fp32 FMA path (batches of up to 4 rows); on the split-bf16
    # MFMA path (5 rows and more) it is w_hi + w_lo, within 2^-16 |w| of w.
    n, k = 40, 512
    w = synth.q5k_weights(n, k, seed=3)
    W = oracle.q5k_dequant_f32(w, n, k)
    wd = dev(w)
    cols = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 300, 511]
    x = np.zeros((len(cols), k), np.float32)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    for i0 in range(0, len(cols), 4):
        y = q4k.q5k_gemv(wd, dev(x[i0:i0 + 4])).cpu().numpy()
        for i, c in enumerate(cols[i0:i0 + 4]):
            assert np.array_equal(y[i], W[:, c]), c
    y = q4k.q5k_gemv(wd, dev(x)).cpu().numpy()
    for i, c in enumerate(cols):
        err = np.abs(y[i].astype(np.float64) - W[:, c])
        assert np.all(err <= 2.0 ** -16 * np.abs(W[:, c])), c


GEMM_TOL = 1e-2


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


# Batches of at most 32 rows (one 32-row slice, split K) and larger ones
# (128 x 128 tiles, split K when the grid is small): ragged M, N and K steps.
@pytest.mark.parametrize("m,n,k", [(1, 256, 512), (8, 520, 1024), (32, 384, 256),
                                   (100, 300, 512), (129, 256, 768)])
def test_q5k_gemm_full_output(q4k, m, n, k):
    w = synth.q5k_weights(n, k, seed=m + n)
    xb = synth.normal_bf16((m, k), seed=m + n)
    Y = q4k.q5k_gemm(dev(w), dev_bf16(xb)).cpu().numpy()
    Yr, A = oracle.q5k_gemm(w, xb, n, k)
    assert_within(Y, Yr, A, GEMM_TOL, "q5k gemm %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k", [(512, 4096, 4096), (16, 14336, 4096)])
def test_q5k_gemm_sampled(q4k, m, n, k):
    w = synth.q5k_weights(n, k, seed=1)
    xb = synth.normal_bf16((m, k), seed=1)
    Y = q4k.q5k_gemm(dev(w), dev_bf16(xb)).cpu().numpy()
    cols = np.unique(np.concatenate([[0, 1, 127, 128, n - 1],
                                     np.random.default_rng(n).integers(0, n, 43)]))
    Yr, A = oracle.q5k_gemm_cols(w, xb, n, k, cols)
    assert_within(Y[:, cols], Yr, A, GEMM_TOL, "q5k gemm %dx%dx%d" % (m, n, k))
    assert np.all(np.isfinite(Y))


def test_q5k_gemm_m1_equals_bf16_weight_dot(q4k):
    # With X exactly representable, the GEMM at m=1 is the dot of X with the
    # bf16 weights the GPU exports (tighter than 1e-2).
    n, k = 256, 2048
    w = synth.q5k_weights(n, k, seed=30)
    xb = synth.normal_bf16((1, k), seed=30)
    Y = q4k.q5k_gemm(dev(w), dev_bf16(xb)).cpu().numpy().astype(np.float64)
    Wb = oracle.q5k_dequant_bf16(w, n, k)
    Wf = (Wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(Y - Xf @ Wf.T) <= 1e-5 * (np.abs(Xf) @ np.abs(Wf.T)))


def test_q5k_gemv_multi_chunk_k(q4k):
    n, k = 300, 20480
    w = synth.q5k_weights(n, k, seed=6)
    x = synth.normal_f32(k, seed=6)
    y = q4k.q5k_gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.q5k_gemv(w, x, n, k)
    assert_within(y, yr[0], a[0], GEMV_TOL, "q5k gemv 300x20480")


@pytest.mark.parametrize("m,n,k", [(6, 8200, 512), (17, 40, 1280), (32, 4096, 1024)])
def test_q5k_gemv_split_batches(q4k, m, n, k):
    # batches of 5..32 rows take the split-bf16 MFMA kernel
    w = synth.q5k_weights(n, k, seed=m + 3)
    x = synth.normal_f32((m, k), seed=m + 3)
    y = q4k.q5k_gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.q5k_gemv(w, x, n, k)
    assert_within(y, yr, a, GEMV_TOL, "q5k split gemv m=%d %dx%d" % (m, n, k))


# Grids that take the streaming kernel on 176-byte records (m <= 32 with at
# least 128 weight tiles of 64 rows; X staged for 8, 16 or 32 rows, 1 to 9
# super-blocks so that some waves have none or an odd count) and the K-slice
# kernels (m > 32 with at least 192 tiles of 64 x 128, else of 64 x 64; ragged
# M and N tiles).  The result is the dot of the bf16 X with the bf16 weights
# of the dequant export, up to fp32 summation order.
@pytest.mark.parametrize("m,n,k", [(1, 8192, 1024), (5, 8200, 512), (8, 8192, 256),
                                   (9, 8200, 1280), (16, 8192, 2304), (17, 9000, 768),
                                   (32, 8192, 768), (330, 4000, 512), (384, 4096, 256),
                                   (256, 4096, 512), (129, 6000, 256)])
def test_q5k_gemm_bf16_weight_dot(q4k, m, n, k):
    w = synth.q5k_weights(n, k, seed=m + 7)
    xb = synth.normal_bf16((m, k), seed=m + 7)
    Y = q4k.q5k_gemm(dev(w), dev_bf16(xb)).cpu().numpy().astype(np.float64)
    Wb = oracle.q5k_dequant_bf16(w, n, k)
    Wf = (Wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert_within(Y, Xf @ Wf.T, np.abs(Xf) @ np.abs(Wf.T), 1e-5, "q5k gemm %dx%dx%d" % (m, n, k))
    if m <= 32:
        Yr, A = oracle.q5k_gemm(w, xb, n, k)
        assert_within(Y, Yr, A, GEMM_TOL, "q5k gemm %dx%dx%d vs oracle" % (m, n, k))
