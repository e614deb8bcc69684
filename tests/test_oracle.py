"""Pins of the CPU oracle (``oracle/``) to facts fixed outside the oracle.

Each test ties one part of the oracle to something it cannot agree with by
accident: a library routine (numpy's binary16 decoder, torch's bf16 rounding,
numpy/scipy matmul and expit), a closed form of the method, a value worked out
by hand (tests/golden/hand_blocks.txt), an exhaustive round trip through an
independently written encoder, or brute force over tiny inputs.  All run on
the CPU.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import synth
from golden_io import hand_blocks
from q4k_pack import f16_bits, pack_block, pack_quants, pack_scales, random_fields


# ---------------------------------------------------------------- binary16

def test_f16_decoder_matches_numpy_exhaustively():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros decode with their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("bits,value", [
    (0x3C00, 1.0), (0x3800, 0.5), (0x4000, 2.0), (0xC000, -2.0),
    (0x0001, 2.0 ** -24), (0x03FF, 1023 * 2.0 ** -24), (0x0400, 2.0 ** -14),
    (0x7BFF, 65504.0), (0x7C00, math.inf), (0x0000, 0.0),
])
def test_f16_closed_form(bits, value):
    assert oracle.f16_to_f64(bits) == value


# ---------------------------------------------------------------- bf16

def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(123)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32),
        (g.standard_normal(2000) * 1e-38).astype(np.float32),  # subnormals
        # exact ties: 7 kept fraction bits, the dropped half is 0x8000
        ((g.integers(0, 2 ** 16, 2000, dtype=np.uint32) << 16) | 0x8000)
        .astype(np.uint32).view(np.float32),
        np.array([0.0, -0.0, 1.0, 65504.0, 3.3895313892515355e38], np.float32),
    ])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_ties_to_even_by_hand():
    # bf16 keeps 7 fraction bits: the ulp at 1.0 is 2^-7.
    assert oracle.f32_to_bf16(1.0 + 2.0 ** -8) == 0x3F80          # tie -> even (1.0)
    assert oracle.f32_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82      # tie -> even (1+2^-6)
    assert oracle.f32_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -20) == 0x3F81
    assert oracle.bf16_to_f64(0x3F81) == 1.0 + 2.0 ** -7
    assert oracle.bf16_to_f64(0xC000) == -2.0


# ---------------------------------------------------------------- format

def test_scale_unpack_roundtrip_every_field_and_value():
    g = np.random.default_rng(1)
    for which in ("sc", "mn"):
        for j in range(8):
            for v in range(64):
                sc = g.integers(0, 64, 8)
                mn = g.integers(0, 64, 8)
                (sc if which == "sc" else mn)[j] = v
                got_sc, got_mn = oracle.unpack_scales(pack_scales(sc, mn))
                assert np.array_equal(got_sc, sc) and np.array_equal(got_mn, mn)


def test_quant_map_roundtrip_every_position_and_value():
    g = np.random.default_rng(2)
    for i in range(256):
        for v in range(16):
            q = g.integers(0, 16, 256)
            q[i] = v
            qs = pack_quants(q)
            assert oracle.quant(qs, i) == v
    q = g.integers(0, 16, 256)
    qs = pack_quants(q)
    assert [oracle.quant(qs, i) for i in range(256)] == list(q)


@pytest.mark.parametrize("name", ["A", "B", "C", "D", "E"])
def test_hand_packed_blocks(name):
    blk, expect = hand_blocks()[name]
    got = oracle.dequant_block(blk).astype(np.float64)
    assert np.array_equal(got, expect), np.nonzero(got != expect)


def test_packer_agrees_with_hand_block_a():
    blk, _ = hand_blocks()["A"]
    q = np.tile(np.array([1] * 32 + [2] * 32), 4)
    mine = pack_block(0x3C00, 0x3800, [1, 2, 3, 4, 0, 0, 0, 0], [5, 6, 7, 8, 0, 0, 0, 0], q)
    assert np.array_equal(mine, blk)


# ---------------------------------------------------------------- closed forms

def test_zero_quants_give_minus_dmin_m():
    g = np.random.default_rng(3)
    for _ in range(200):
        d, dmin, sc, mn, _q = random_fields(g)
        w = oracle.dequant_block(pack_block(d, dmin, sc, mn, np.zeros(256, int)))
        dm = np.float16(np.uint16(dmin).view(np.float16)).astype(np.float64)
        for j in range(8):
            assert np.all(w[32 * j: 32 * j + 32] == np.float32(-dm * mn[j]))


def test_constant_quants_closed_form():
    g = np.random.default_rng(4)
    for c in range(16):
        d, dmin, sc, mn, _q = random_fields(g)
        w = oracle.dequant_block(pack_block(d, dmin, sc, mn, np.full(256, c)))
        dd = np.uint16(d).view(np.float16).astype(np.float64)
        dm = np.uint16(dmin).view(np.float16).astype(np.float64)
        for j in range(8):
            assert np.all(w[32 * j: 32 * j + 32] == np.float32(dd * sc[j] * c - dm * mn[j]))


def test_dequant_is_exact_rounding_of_rational_value():
    # brute force with exact rationals on random blocks, subnormal scales included
    from fractions import Fraction
    g = np.random.default_rng(5)
    for trial in range(40):
        d, dmin, sc, mn, q = random_fields(g)
        if trial % 4 == 0:
            d = int(g.integers(1, 1024))        # subnormal d
        if trial % 4 == 1:
            dmin = int(g.integers(1, 1024))     # subnormal dmin
        w = oracle.dequant_block(pack_block(d, dmin, sc, mn, q))
        dd = Fraction(float(np.uint16(d).view(np.float16)))
        dm = Fraction(float(np.uint16(dmin).view(np.float16)))
        for i in range(0, 256, 7):
            exact = dd * int(sc[i // 32]) * int(q[i]) - dm * int(mn[i // 32])
            # float32(float(exact)) is a double rounding only if float(exact) rounds;
            # exact fits in 53 bits here, so float(exact) is exact.
            assert Fraction(float(exact)) == exact
            assert w[i] == np.float32(float(exact))


def test_random_matrix_dequant_vs_packer_fields():
    # a full random matrix from the generator, decoded through the oracle, against
    # per-block decoding of the same bytes
    n, k = 4, 512
    w = synth.q4k_weights(n, k, seed=7)
    full = oracle.dequant_f32(w, n, k)
    blocks = w.reshape(-1, 144)
    per = np.concatenate([oracle.dequant_block(b) for b in blocks]).reshape(n, k)
    assert np.array_equal(full, per)


def test_dequant_bf16_is_rne_of_f32():
    n, k = 8, 1024
    w = synth.q4k_weights(n, k, seed=8)
    f = oracle.dequant_f32(w, n, k)
    b = oracle.dequant_bf16(w, n, k)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


# ---------------------------------------------------------------- GEMV

def test_gemv_unit_vectors_give_columns():
    # y(e_k) = column k of W: pins the k -> (block, sub-block, nibble) map and
    # the orientation of the product
    n, k = 6, 512
    w = synth.q4k_weights(n, k, seed=9)
    eye = np.eye(k, dtype=np.float32)
    y, a = oracle.gemv(w, eye, n, k)
    W = oracle.dequant_f32(w, n, k)
    assert np.array_equal(y, W.T.astype(np.float64))
    assert np.array_equal(a, np.abs(W.T.astype(np.float64)))


def test_gemv_matches_library_matmul():
    n, k = 64, 1024
    w = synth.q4k_weights(n, k, seed=10)
    x = synth.normal_f32((3, k), seed=10)
    y, a = oracle.gemv(w, x, n, k)
    W = oracle.dequant_f32(w, n, k).astype(np.float64)
    ref = x.astype(np.float64) @ W.T
    assert np.all(np.abs(y - ref) <= 1e-12 * a)
    assert np.allclose(a, np.abs(x.astype(np.float64)) @ np.abs(W.T))


def test_gemv_is_linear_in_x():
    n, k = 16, 768
    w = synth.q4k_weights(n, k, seed=11)
    g = np.random.default_rng(11)
    # small integers: alpha*x1 + beta*x2 is exact in fp32
    x1 = g.integers(-50, 50, k).astype(np.float32)
    x2 = g.integers(-50, 50, k).astype(np.float32)
    y1, a1 = oracle.gemv(w, x1, n, k)
    y2, a2 = oracle.gemv(w, x2, n, k)
    y3, _ = oracle.gemv(w, 3 * x1 - 2 * x2, n, k)
    assert np.all(np.abs(y3 - (3 * y1 - 2 * y2)) <= 1e-12 * (3 * a1 + 2 * a2))


def test_gemv_row_constant_fields_reduce_to_subblock_sums():
    # every block identical with constant quant c: y = sum_j (d sc_j c - dmin m_j) S_j
    g = np.random.default_rng(12)
    d, dmin, sc, mn, _ = random_fields(g)
    c = 9
    blk = pack_block(d, dmin, sc, mn, np.full(256, c))
    n, k = 3, 1024
    w = np.tile(blk, n * k // 256).reshape(n, -1)
    x = synth.normal_f32(k, seed=12)
    y, _ = oracle.gemv(w, x, n, k)
    dd = np.uint16(d).view(np.float16).astype(np.float64)
    dm = np.uint16(dmin).view(np.float16).astype(np.float64)
    S = x.astype(np.float64).reshape(-1, 8, 32).sum(axis=2)  # [blocks, sub-blocks]
    vals = np.array([np.float32(dd * sc[j] * c - dm * mn[j]) for j in range(8)], np.float64)
    expect = (S * vals[None, :]).sum()
    assert np.allclose(y, expect, rtol=1e-12, atol=1e-12)


def test_gemv_rows_subset_equals_full():
    n, k = 40, 512
    w = synth.q4k_weights(n, k, seed=13)
    x = synth.normal_f32((2, k), seed=13)
    y, a = oracle.gemv(w, x, n, k)
    rows = [0, 7, 39, 13]
    ys, as_ = oracle.gemv_rows(w, x, n, k, rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(as_, a[:, rows])


def test_bad_shapes_rejected():
    w = synth.q4k_weights(2, 256, seed=0)
    with pytest.raises(ValueError):
        oracle.gemv_rows(w, np.zeros(256, np.float32), 2, 256, [2])


# ---------------------------------------------------------------- GEMM

def test_gemm_at_m1_with_bf16_exact_x_equals_gemv():
    n, k = 32, 1024
    w = synth.q4k_weights(n, k, seed=14)
    xb = synth.normal_bf16((1, k), seed=14)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    y1, a1 = oracle.gemm(w, xb, n, k)
    y2, a2 = oracle.gemv(w, xf, n, k)
    assert np.array_equal(y1, y2) and np.array_equal(a1, a2)


def test_gemm_matches_library_matmul():
    m, n, k = 9, 24, 512
    w = synth.q4k_weights(n, k, seed=15)
    xb = synth.normal_bf16((m, k), seed=15)
    X = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    W = oracle.dequant_f32(w, n, k).astype(np.float64)
    y, a = oracle.gemm(w, xb, n, k)
    assert np.all(np.abs(y - X @ W.T) <= 1e-12 * a)
    cols = [23, 0, 5]
    yc, ac = oracle.gemm_cols(w, xb, n, k, cols)
    assert np.array_equal(yc, y[:, cols]) and np.array_equal(ac, a[:, cols])


# ---------------------------------------------------------------- SiLU / MLP

def test_silu_identities():
    assert oracle.silu(0.0) == 0.0
    for t in [0.1, 1.0, 2.5, 7.0, 30.0]:
        # silu(t) - silu(-t) = t sigma(t) + t sigma(t) - t = t (sigma(t) + sigma(-t) = 1)
        assert abs(oracle.silu(t) - oracle.silu(-t) - t) <= 1e-15 * max(1.0, t)
        assert abs(oracle.silu(t) - t * expit(t)) <= 1e-15 * t
    v = oracle.silu(-100.0)
    assert v < 0 and abs(v - (-100.0 * math.exp(-100.0))) <= 1e-15 * abs(v)
    assert abs(oracle.silu(50.0) - 50.0) < 1e-15 * 50


def test_swiglu_mlp_matches_library_composition():
    dm, dff = 256, 512
    wg = synth.q4k_weights(dff, dm, seed=16, stream=synth.W_GATE)
    wu = synth.q4k_weights(dff, dm, seed=16, stream=synth.W_UP)
    wd = synth.q4k_weights(dm, dff, seed=16, stream=synth.W_DOWN)
    x = synth.normal_f32(dm, seed=16) * 4
    r = oracle.swiglu_mlp(wg, wu, wd, x, dm, dff)
    G = oracle.dequant_f32(wg, dff, dm).astype(np.float64)
    U = oracle.dequant_f32(wu, dff, dm).astype(np.float64)
    D = oracle.dequant_f32(wd, dm, dff).astype(np.float64)
    g = G @ x.astype(np.float64)
    u = U @ x.astype(np.float64)
    h = g * expit(g) * u
    out = D @ h
    assert np.all(np.abs(r["g"] - g) <= 1e-12 * (np.abs(G) @ np.abs(x.astype(np.float64))))
    assert np.allclose(r["h"], h, rtol=1e-12, atol=1e-14)
    assert np.all(np.abs(r["out"] - out) <= 1e-11 * (np.abs(D) @ np.abs(h)) + 1e-14)
    assert np.allclose(r["aout"], np.abs(D) @ np.abs(r["h"]), rtol=1e-12)
    # the GEMV of W_down against the same h reproduces out (down = GEMV stage)
    yd, _ = oracle.gemv(wd, r["h"].astype(np.float32), dm, dff)
    assert np.allclose(yd[0], out, rtol=1e-5, atol=1e-6 * np.abs(out).max())


# ---------------------------------------------------------------- Q5_K oracle

Q5K_HAND = hand_blocks("hand_blocks_q5k.txt", block_bytes=176)


@pytest.mark.parametrize("name", sorted(Q5K_HAND))
def test_q5k_hand_packed_blocks(name):
    blk, expected = Q5K_HAND[name]
    got = oracle.q5k_dequant_block(blk).astype(np.float64)
    assert np.array_equal(got, expected), name


def test_q5k_with_clear_high_bits_equals_q4k():
    # With every fifth bit clear a Q5_K block is the Q4_K block with the same
    # scales and nibbles: ties the Q5_K decoder to the pinned Q4_K one.
    w4 = synth.q4k_weights(64, 256, seed=11)
    for b4 in w4:
        b5 = np.concatenate([b4[:16], np.zeros(32, np.uint8), b4[16:]])
        assert np.array_equal(oracle.q5k_dequant_block(b5).view(np.uint32),
                              oracle.dequant_block(b4).view(np.uint32))


def test_q5k_high_bit_map_every_bit():
    # One high bit at a time (d = 1, dmin = 0, sc = 1, nibbles 0): exactly the
    # weight 64 (u div 2) + 32 (u mod 2) + l of bit u of qh[l] becomes 16.
    base = np.zeros(176, np.uint8)
    base[1] = 0x3C
    base[4:8] = 1
    base[12:16] = 1
    for l in range(32):
        for u in range(8):
            blk = base.copy()
            blk[16 + l] = 1 << u
            w = oracle.q5k_dequant_block(blk)
            want = np.zeros(256, np.float32)
            want[64 * (u // 2) + 32 * (u % 2) + l] = 16.0
            assert np.array_equal(w, want), (l, u)


def test_q5k_quant_roundtrip_every_position_and_value():
    from q5k_pack import pack_high_bits
    from q4k_pack import pack_quants
    for v in range(32):
        for i in range(256):
            q = np.zeros(256, np.int64)
            q[i] = v
            qh, qs = pack_high_bits(q), pack_quants(q % 16)
            assert oracle.q5k_quant(qh, qs, i) == v
            if v:
                j = (i + 97) % 256
                assert oracle.q5k_quant(qh, qs, j) == 0


def test_q5k_zero_quants_give_minus_dmin_m():
    from q5k_pack import pack_q5k_block
    sc = [3, 7, 0, 63, 1, 2, 40, 5]
    mn = [9, 0, 63, 4, 33, 1, 6, 17]
    blk = pack_q5k_block(0x3C00, 0x3555, sc, mn, np.zeros(256, np.int64))
    dmin = float(np.array([0x3555], np.uint16).view(np.float16)[0])
    want = np.repeat([np.float32(-dmin * m) for m in mn], 32)
    assert np.array_equal(oracle.q5k_dequant_block(blk), want)


def test_q5k_dequant_bf16_is_rne_of_f32():
    w = synth.q5k_weights(16, 512, seed=4)
    f = oracle.q5k_dequant_f32(w, 16, 512)
    b = oracle.q5k_dequant_bf16(w, 16, 512)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_q5k_gemv_unit_vectors_give_columns():
    n, k = 24, 512
    w = synth.q5k_weights(n, k, seed=8)
    W = oracle.q5k_dequant_f32(w, n, k).astype(np.float64)
    for c in (0, 1, 31, 32, 63, 64, 255, 256, 300, 511):
        x = np.zeros(k, np.float32)
        x[c] = 1.0
        y, _ = oracle.q5k_gemv(w, x, n, k)
        assert np.array_equal(y[0], W[:, c])


def test_q5k_gemv_matches_library_matmul():
    n, k, m = 40, 768, 3
    w = synth.q5k_weights(n, k, seed=12)
    x = synth.normal_f32((m, k), seed=12)
    y, a = oracle.q5k_gemv(w, x, n, k)
    W = oracle.q5k_dequant_f32(w, n, k).astype(np.float64)
    ref = x.astype(np.float64) @ W.T
    assert np.all(np.abs(y - ref) <= 1e-12 * a)
    assert np.allclose(a, np.abs(x.astype(np.float64)) @ np.abs(W.T))
    rows = np.array([0, 7, 39])
    yr, ar = oracle.q5k_gemv_rows(w, x, n, k, rows)
    assert np.array_equal(yr, y[:, rows]) and np.array_equal(ar, a[:, rows])


def test_q5k_bad_shapes_rejected():
    w = synth.q5k_weights(2, 256, seed=0)
    L = oracle.lib()
    out = np.zeros(512, np.float32)
    assert L.oracle_q5k_dequant_f32(oracle._p(w, oracle._u8p), 2, 300,
                                    oracle._p(out, oracle._f32p)) == -1


def test_q5k_gemm_at_m1_with_bf16_exact_x_equals_gemv():
    n, k = 20, 512
    w = synth.q5k_weights(n, k, seed=21)
    xb = synth.normal_bf16((1, k), seed=21)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    y, a = oracle.q5k_gemm(w, xb, n, k)
    yv, av = oracle.q5k_gemv(w, xf, n, k)
    assert np.array_equal(y, yv) and np.array_equal(a, av)


def test_q5k_gemm_matches_library_matmul():
    n, k, m = 24, 512, 5
    w = synth.q5k_weights(n, k, seed=22)
    xb = synth.normal_bf16((m, k), seed=22)
    Xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    W = oracle.q5k_dequant_f32(w, n, k).astype(np.float64)
    y, a = oracle.q5k_gemm(w, xb, n, k)
    assert np.all(np.abs(y - Xf @ W.T) <= 1e-12 * a)
    cols = np.array([3, 0, 23])
    yc, ac = oracle.q5k_gemm_cols(w, xb, n, k, cols)
    assert np.array_equal(yc, y[:, cols]) and np.array_equal(ac, a[:, cols])


# ---------------------------------------------------------------- all-cores build

def test_openmp_build_returns_identical_bits():
    # liboracle_omp.so runs whole output rows per thread in the same k order;
    # its results must equal the plain build's bit for bit.
    n, k, m = 96, 1024, 3
    w = synth.q4k_weights(n, k, seed=41)
    x = synth.normal_f32((m, k), seed=41)
    y1, a1 = oracle.gemv(w, x, n, k)
    y2, a2 = oracle.gemv(w, x, n, k, omp=True)
    assert np.array_equal(y1, y2) and np.array_equal(a1, a2)
    xb = synth.normal_bf16((m, k), seed=41)
    cols = np.arange(0, n, 5)
    g1, b1 = oracle.gemm_cols(w, xb, n, k, cols)
    g2, b2 = oracle.gemm_cols(w, xb, n, k, cols, omp=True)
    assert np.array_equal(g1, g2) and np.array_equal(b1, b2)
    dm, dff = 256, 512
    wg = synth.q4k_weights(dff, dm, seed=42, stream=synth.W_GATE)
    wu = synth.q4k_weights(dff, dm, seed=42, stream=synth.W_UP)
    wd = synth.q4k_weights(dm, dff, seed=42, stream=synth.W_DOWN)
    xm = synth.normal_f32(dm, seed=42)
    r1 = oracle.swiglu_mlp(wg, wu, wd, xm, dm, dff)
    r2 = oracle.swiglu_mlp(wg, wu, wd, xm, dm, dff, omp=True)
    for key in r1:
        assert np.array_equal(r1[key], r2[key]), key
    assert oracle.threads() == 1 and oracle.threads(omp=True) >= 1
