"""Parity of the Q3_K entry points (q3k_gemv, q3k_dequantize_*) with the oracle.

Same bars as Q4_K: dequantized weights bit-exact (fp32, and bf16 = nearest
even of fp32); GEMV within 1e-4 * sum|w x| per output.  Shapes cover blocks
that start 2 bytes past a dword boundary (odd block counts per row), ragged
row tiles (n not a multiple of 16), K past one 4096-wide x chunk, batches, and
the hand-packed blocks.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from golden_io import hand_blocks

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


def check_dequant(q4k, w, n, k):
    got = q4k.q3k_dequantize_f32(dev(w)).cpu().numpy()
    ref = oracle.q3k_dequant_f32(w, n, k)
    bad = got.view(np.uint32) != ref.view(np.uint32)
    assert not bad.any(), "%d of %d weights differ, first at %s" % (bad.sum(), bad.size,
                                                                   np.argwhere(bad)[:3].tolist())
    got16 = q4k.q3k_dequantize_bf16(dev(w)).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got16, oracle.q3k_dequant_bf16(w, n, k))


@pytest.mark.parametrize("n,k,seed", [(256, 1024, 0), (37, 768, 1), (3, 256, 2), (4096, 4096, 0)])
def test_q3k_dequant_bit_exact(q4k, n, k, seed):
    check_dequant(q4k, synth.q3k_weights(n, k, seed=seed), n, k)


def test_q3k_dequant_hand_blocks(q4k):
    blocks = hand_blocks("hand_blocks_q3k.txt", block_bytes=110)
    names = sorted(blocks)
    w = np.concatenate([blocks[nm][0] for nm in names]).reshape(1, -1)  # one row, 4 blocks
    k = 256 * len(names)
    got = q4k.q3k_dequantize_f32(dev(w)).cpu().numpy().reshape(-1)
    for i, nm in enumerate(names):
        np.testing.assert_array_equal(got[256 * i: 256 * (i + 1)].astype(np.float64), blocks[nm][1])
    check_dequant(q4k, w, 1, k)


def assert_within(got, ref, scale, what):
    err = np.abs(np.asarray(got, np.float64) - ref)
    bad = err > GEMV_TOL * scale
    assert not bad.any(), "%s: %d outputs outside 1e-4 * sum|w x|, worst %g" % (
        what, bad.sum(), (err / np.maximum(GEMV_TOL * scale, 1e-300)).max())


@pytest.mark.parametrize("n,k,m,seed", [
    (256, 1024, 1, 0),
    (4096, 4096, 1, 1),     # the decode shape
    (37, 768, 1, 2),        # odd blocks per row, ragged row tile
    (100, 8448, 1, 3),      # three x chunks, the last one block wide
    (14336, 4096, 1, 4),    # tall
    (300, 1280, 3, 5),      # a batch (one pass of up to 4 x rows)
    (64, 512, 5, 7),        # two passes: 4 + 1
    (50, 4352, 8, 8),       # two full passes, x past one chunk
    (17, 256, 2, 9),        # a pass of 2
    # rows staged through LDS (n * k / 256 a multiple of 8) that start at
    # varying offsets mod 16: two chunks, the last one block wide; a batch
    (8, 4352, 1, 10),
    (24, 8448, 3, 11),
    (40, 1280, 2, 12),
])
def test_q3k_gemv(q4k, n, k, m, seed):
    w = synth.q3k_weights(n, k, seed=seed)
    x = synth.normal_f32((m, k), seed=seed)
    y = q4k.q3k_gemv(dev(w), dev(x)).cpu().numpy()
    if n * k <= 4096 * 4096:
        yr, a = oracle.q3k_gemv(w, x, n, k)
    else:
        rows = np.arange(0, n, 7)
        yr, a = oracle.q3k_gemv_rows(w, x, n, k, rows)
        y = y[:, rows]
    assert_within(y, yr, a, "q3k_gemv %dx%d m=%d" % (n, k, m))


def test_q3k_gemv_unit_vectors(q4k):
    n, k = 64, 1024
    w = synth.q3k_weights(n, k, seed=6)
    W = oracle.q3k_dequant_f32(w, n, k)
    for c in (0, 31, 32, 255, 256, 767, 1023):
        x = np.zeros(k, np.float32)
        x[c] = 1.0
        y = q4k.q3k_gemv(dev(w), dev(x)).cpu().numpy()
        np.testing.assert_allclose(y, W[:, c], rtol=0, atol=1e-6 * np.abs(W[:, c]).max())



def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("m,n,k", [(1, 128, 256), (8, 520, 1024), (32, 384, 768), (64, 200, 512),
                                   (130, 257, 1280), (130, 264, 1280), (300, 136, 2048)])
def test_q3k_gemm_full_output(q4k, m, n, k):
    # split-K grids (small tiles) and full ones, ragged tiles, odd block counts per row; for m > 32
    # the operands go through LDS by copies when n * k / 256 is a multiple of 8 (64 x 200, 130 x
    # 264 with 5 super-blocks split 3 + 2, 300 x 136 split four ways), else the tile kernel loads
    # them (130 x 257)
    w = synth.q3k_weights(n, k, seed=m + n)
    xb = synth.normal_bf16((m, k), seed=m + n)
    y = q4k.q3k_gemm(dev(w), _dev_bf16(xb)).cpu().numpy()
    ref, a = oracle.q3k_gemm(w, xb, n, k)
    err = np.abs(y - ref)
    assert (err <= 1e-2 * a).all(), "q3k_gemm %dx%dx%d: worst %g" % (m, n, k, (err / (1e-2 * a)).max())


def test_q3k_gemm_prefill_shape_sampled(q4k):
    m, n, k = 512, 4096, 4096
    w = synth.q3k_weights(n, k, seed=3)
    xb = synth.normal_bf16((m, k), seed=3)
    y = q4k.q3k_gemm(dev(w), _dev_bf16(xb)).cpu().numpy()
    cols = np.concatenate([np.arange(0, n, 97), [n - 1]])
    ref, a = oracle.q3k_gemm_cols(w, xb, n, k, cols)
    assert (np.abs(y[:, cols] - ref) <= 1e-2 * a).all()
