"""Pins of the Q6_K oracle to facts fixed outside it.

The oracle (``oracle/q6k_oracle.c``) follows the Q6_K reading documented in
its header (the daScript PR page names the 6-bit k-quant, its high-bit plane
and per-sub-block scales, and prints no layout).  Pins: hand-packed blocks with
hand-computed weights, round trips through an independently written test
encoder, every position and value of the 6-bit quant, closed forms (q = 32
gives zero, q = 0 gives -32 d sc), and the GEMV against unit vectors and numpy.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from golden_io import hand_blocks
from q6k_pack import pack_q6k_block

Q6K_HAND = hand_blocks("hand_blocks_q6k.txt", block_bytes=210)


@pytest.mark.parametrize("name", sorted(Q6K_HAND))
def test_q6k_hand_packed_blocks(name):
    blk, expected = Q6K_HAND[name]
    got = oracle.q6k_dequant_block(blk).astype(np.float64)
    np.testing.assert_array_equal(got, expected)


def test_q6k_quant_every_position_and_value():
    rng = np.random.default_rng(3)
    for i in range(256):
        for v in (1, 15, 16, 31, 32, 48, 63):
            q = np.zeros(256, np.int64)
            q[i] = v
            blk = pack_q6k_block(0x3C00, np.ones(16), q)
            assert oracle.q6k_quant(blk, i) == v
            others = [j for j in rng.choice(256, 8, replace=False) if j != i]
            for j in others:
                assert oracle.q6k_quant(blk, j) == 0


def test_q6k_random_round_trip():
    rng = np.random.default_rng(5)
    for _ in range(20):
        q = rng.integers(0, 64, 256)
        sc = rng.integers(-128, 128, 16)
        blk = pack_q6k_block(0x3C00, sc, q)  # d = 1
        w = oracle.q6k_dequant_block(blk).astype(np.float64)
        np.testing.assert_array_equal(w, np.repeat(sc, 16) * (q - 32.0))
        assert [oracle.q6k_quant(blk, i) for i in range(256)] == q.tolist()


def test_q6k_closed_forms():
    sc = np.arange(-8, 8) * 9
    # q = 32 everywhere: every weight is zero
    w = oracle.q6k_dequant_block(pack_q6k_block(0x3555, sc, np.full(256, 32)))
    assert not w.any()
    # q = 0 everywhere: -32 d sc, with d = 0x3555 = 0.333251953125
    w = oracle.q6k_dequant_block(pack_q6k_block(0x3555, sc, np.zeros(256, np.int64)))
    want = (np.repeat(sc, 16) * -32 * 0.333251953125).astype(np.float32)
    np.testing.assert_array_equal(w, want)


def test_q6k_single_rounding_of_a_wide_product():
    # d = 2047/1024 (11 significant bits), sc = 127, q - 32 = 31: the exact product
    # 2047 * 127 * 31 / 1024 needs 24 bits -- exactly representable; q - 32 = -31 and
    # sc = -127 give the same magnitude.  A subnormal d (0x0001 = 2^-24) stays exact too.
    q = np.full(256, 63)
    w = oracle.q6k_dequant_block(pack_q6k_block(0x3FFF, np.full(16, 127), q))
    assert (w.astype(np.float64) == 2047 * 127 * 31 / 1024).all()
    w = oracle.q6k_dequant_block(pack_q6k_block(0x0001, np.full(16, -128), np.zeros(256, np.int64)))
    assert (w.astype(np.float64) == 2.0 ** -24 * -128 * -32).all()


def test_q6k_dequant_bf16_is_rne_of_f32():
    w = synth.q6k_weights(16, 512, seed=4)
    f = oracle.q6k_dequant_f32(w, 16, 512)
    b = oracle.q6k_dequant_bf16(w, 16, 512)
    np.testing.assert_array_equal(b, synth.bf16_bits(f))


def test_q6k_rows_are_consecutive_blocks():
    w = synth.q6k_weights(3, 768, seed=6)
    f = oracle.q6k_dequant_f32(w, 3, 768)
    for r in range(3):
        for b in range(3):
            blk = w[r, 210 * b: 210 * (b + 1)]
            np.testing.assert_array_equal(f[r, 256 * b: 256 * (b + 1)], oracle.q6k_dequant_block(blk))


def test_q6k_gemv_unit_vectors_give_columns():
    n, k = 8, 512
    w = synth.q6k_weights(n, k, seed=8)
    W = oracle.q6k_dequant_f32(w, n, k).astype(np.float64)
    for c in (0, 1, 255, 256, 511):
        x = np.zeros(k, np.float32)
        x[c] = 1.0
        y, _ = oracle.q6k_gemv(w, x, n, k)
        np.testing.assert_array_equal(y[0], W[:, c])


def test_q6k_gemv_matches_library_matmul():
    n, k, m = 24, 1024, 3
    w = synth.q6k_weights(n, k, seed=9)
    x = synth.normal_f32((m, k), seed=9)
    y, a = oracle.q6k_gemv(w, x, n, k)
    W = oracle.q6k_dequant_f32(w, n, k).astype(np.float64)
    ref = x.astype(np.float64) @ W.T
    assert np.all(np.abs(y - ref) <= 1e-12 * a)
    np.testing.assert_allclose(a, np.abs(x.astype(np.float64)) @ np.abs(W).T, rtol=1e-12)
    rows = np.array([23, 0, 7])
    yr, _ = oracle.q6k_gemv_rows(w, x, n, k, rows)
    np.testing.assert_array_equal(yr, y[:, rows])


# ---------------------------------------------------------------- GEMM

def test_q6k_gemm_at_m1_with_bf16_exact_x_equals_gemv():
    # A bf16 row is exactly an fp32 row, so the GEMM at one row must return
    # the GEMV's sums bit for bit (same fp32 weights, same k order).
    n, k = 24, 1024
    w = synth.q6k_weights(n, k, seed=31)
    xb = synth.normal_bf16((1, k), seed=31)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    y1, a1 = oracle.q6k_gemm(w, xb, n, k)
    y2, a2 = oracle.q6k_gemv(w, xf, n, k)
    assert np.array_equal(y1, y2) and np.array_equal(a1, a2)


def test_q6k_gemm_matches_library_matmul():
    import torch
    m, n, k = 7, 20, 768
    w = synth.q6k_weights(n, k, seed=32)
    xb = synth.normal_bf16((m, k), seed=32)
    X = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    W = oracle.q6k_dequant_f32(w, n, k).astype(np.float64)
    y, a = oracle.q6k_gemm(w, xb, n, k)
    assert np.all(np.abs(y - X @ W.T) <= 1e-12 * a)
    np.testing.assert_allclose(a, np.abs(X) @ np.abs(W).T, rtol=1e-12)
    cols = [19, 0, 6]
    yc, ac = oracle.q6k_gemm_cols(w, xb, n, k, cols)
    assert np.array_equal(yc, y[:, cols]) and np.array_equal(ac, a[:, cols])


def test_q6k_gemm_zero_weights_give_exact_zero():
    # A matrix whose weights are all zero gives exactly +-0 with A = 0.
    n, k, m = 3, 256, 4
    w = np.zeros((n, k // 256 * oracle.Q6K_BLOCK_BYTES), np.uint8)
    xb = synth.normal_bf16((m, k), seed=33)
    y, a = oracle.q6k_gemm(w, xb, n, k)
    assert np.all(y == 0.0) and np.all(a == 0.0)
