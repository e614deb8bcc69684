"""Structured blocks through every compute path, element by element against the oracle.

The seeded matrices of the other parity tests never exercise the format's
degenerate cases inside the GEMV, GEMM and MLP kernels.  Here every matrix is
tiled from hand-made blocks:
  * the hand-packed golden blocks (weights worked out by hand);
  * zero quants (every weight -dmin m, the closed form of the target) and
    constant quants (d sc c - dmin m);
  * subnormal and largest-finite fp16 d / dmin, zero scales;
  * blocks whose weights cancel exactly to zero (d sc q = dmin m for every
    weight, with one or several scale pairs), and blocks that nearly cancel
    (|w| a thousandth of dmin m, or zero but for a few +-1 weights).
Rows built only from cancelling blocks have sum|w x| = 0, so the bar
|y - y_oracle| <= tol * sum|w x| demands exactly +-0 there; every other output
meets the same bar as the seeded tests (1e-4 for the fp32 GEMVs and the MLP
stages, 1e-2 for the bf16 GEMMs).  The pages ("Writing an ESIMD Fused Kernel
From Reverse-Engineered Assembly", "Getting Q4_K Right"; daScript PR page,
"Validation") check every kernel variant against the reference decode; these
blocks are where a refactored dot would part from it.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from golden_io import hand_blocks
from q3k_pack import pack_q3k_block
from q4k_pack import f16_bits, pack_block
from q5k_pack import pack_q5k_block
from q6k_pack import pack_q6k_block

pytestmark = pytest.mark.gpu

GEMV_TOL = 1e-4
GEMM_TOL = 1e-2
ONE = 0x3C00


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


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def assert_within(got, ref, scale, tol, what):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bound = tol * scale
    bad = err > bound
    if bad.any():
        i = np.argmax(err / np.maximum(bound, 1e-300))
        raise AssertionError("%s: %d outputs outside %g * sum|w x| (%d of them with sum 0); worst "
                             "at %s: got %r ref %r bound %r"
                             % (what, bad.sum(), tol, (bad & (scale == 0)).sum(),
                                np.unravel_index(i, err.shape), got.flat[i], ref.flat[i],
                                bound.flat[i]))


# ------------------------------------------------------------------ block kinds

def q4k_kinds():
    """(cancelling, other) lists of structured 144-byte Q4_K blocks."""
    g = np.random.default_rng(123)
    sc = g.integers(0, 64, 8)
    mn = g.integers(0, 64, 8)
    rq = lambda: g.integers(0, 16, 256)  # noqa: E731
    other = [blk for _, (blk, _) in sorted(hand_blocks().items())]
    other += [
        pack_block(f16_bits(0.013), f16_bits(0.007), sc, mn, np.zeros(256, int)),  # zero quants
        pack_block(f16_bits(0.021), f16_bits(0.004), sc, mn, np.full(256, 9)),  # constant quants
        pack_block(0x0001, 0x03FF, sc, mn, rq()),  # subnormal d and dmin
        pack_block(0x03FF, 0x0001, np.full(8, 63), np.full(8, 63), rq()),
        pack_block(0x7BFF, 0x7BFF, np.full(8, 63), np.full(8, 63), rq()),  # largest finite
        pack_block(ONE, ONE, np.zeros(8, int), np.zeros(8, int), rq()),  # zero scales
        # nearly cancelling: d = 1 + 2^-10, so every weight is 3 * 2^-10
        pack_block(0x3C01, ONE, np.ones(8, int), np.full(8, 3), np.full(256, 3)),
        # cancelling but for three +-1 weights
        pack_block(ONE, ONE, np.ones(8, int), np.full(8, 3),
                   np.where(np.isin(np.arange(256), [5, 77, 200]), [4] * 256, 3)),
        # per sub-block near cancellation: q = 7 against mn = 7 sc + 1
        pack_block(0x3800, 0x3800, np.arange(1, 9), 7 * np.arange(1, 9) - 1, np.full(256, 7)),
    ]
    cancel = [
        pack_block(ONE, ONE, np.ones(8, int), np.full(8, 3), np.full(256, 3)),
        pack_block(ONE, ONE, np.arange(1, 9), 7 * np.arange(1, 9), np.full(256, 7)),
        pack_block(0x3800, 0x3400, np.full(8, 6), np.full(8, 60), np.full(256, 5)),
        pack_block(f16_bits(0.013), f16_bits(0.013), np.full(8, 12), np.full(8, 60),
                   np.full(256, 5)),
        pack_block(0x0000, 0x0000, sc, mn, rq()),  # d = dmin = 0
    ]
    return cancel, other


def q5k_kinds():
    g = np.random.default_rng(124)
    sc = g.integers(0, 64, 8)
    mn = g.integers(0, 64, 8)
    other = [blk for _, (blk, _) in sorted(hand_blocks("hand_blocks_q5k.txt", 176).items())]
    other += [
        pack_q5k_block(f16_bits(0.011), f16_bits(0.006), sc, mn, np.zeros(256, int)),
        pack_q5k_block(f16_bits(0.017), f16_bits(0.003), sc, mn, np.full(256, 25)),
        pack_q5k_block(0x0001, 0x03FF, sc, mn, g.integers(0, 32, 256)),
        pack_q5k_block(0x7BFF, 0x7BFF, np.full(8, 63), np.full(8, 63), g.integers(0, 32, 256)),
        pack_q5k_block(0x3C01, ONE, np.ones(8, int), np.full(8, 19), np.full(256, 19)),
        pack_q5k_block(ONE, ONE, np.ones(8, int), np.full(8, 19),
                       np.where(np.isin(np.arange(256), [3, 130, 255]), [20] * 256, 19)),
    ]
    cancel = [
        pack_q5k_block(ONE, ONE, np.ones(8, int), np.full(8, 19), np.full(256, 19)),  # fifth bit set
        pack_q5k_block(ONE, ONE, np.full(8, 2), np.full(8, 6), np.full(256, 3)),
        pack_q5k_block(0x3800, 0x3400, np.ones(8, int), np.full(8, 62), np.full(256, 31)),
    ]
    return cancel, other


def q6k_kinds():
    g = np.random.default_rng(125)
    sc = g.integers(-128, 128, 16)
    other = [blk for _, (blk, _) in sorted(hand_blocks("hand_blocks_q6k.txt", 210).items())]
    other += [
        pack_q6k_block(f16_bits(2e-4), sc, np.zeros(256, int)),  # q = 0: -32 d sc
        pack_q6k_block(0x0001, sc, g.integers(0, 64, 256)),  # subnormal d
        pack_q6k_block(0x7BFF, np.full(16, 127), g.integers(0, 64, 256)),
        pack_q6k_block(f16_bits(3e-4), sc,
                       np.where(np.isin(np.arange(256), [0, 100, 255]), [33] * 256, 32)),
    ]
    cancel = [
        pack_q6k_block(f16_bits(3e-4), sc, np.full(256, 32)),  # q = 32: every weight zero
        pack_q6k_block(ONE, np.zeros(16, int), g.integers(0, 64, 256)),  # zero scales
        pack_q6k_block(0x0000, sc, g.integers(0, 64, 256)),  # d = 0
    ]
    return cancel, other


def q3k_kinds():
    g = np.random.default_rng(126)
    sc = g.integers(-32, 32, 16)
    other = [blk for _, (blk, _) in sorted(hand_blocks("hand_blocks_q3k.txt", 110).items())]
    other += [
        pack_q3k_block(f16_bits(1e-3), sc, np.full(256, -4)),
        pack_q3k_block(0x0001, sc, g.integers(-4, 4, 256)),
        pack_q3k_block(0x7BFF, np.full(16, -32), g.integers(-4, 4, 256)),
        pack_q3k_block(f16_bits(2e-3), sc,
                       np.where(np.isin(np.arange(256), [1, 128, 254]), [1] * 256, 0)),
    ]
    cancel = [
        pack_q3k_block(f16_bits(2e-3), sc, np.zeros(256, int)),  # q = 0: every weight zero
        pack_q3k_block(ONE, np.zeros(16, int), g.integers(-4, 4, 256)),  # zero scales
    ]
    return cancel, other


def tile(kinds, n, k, seed):
    """[n, k/256 * block] matrix: every third row only cancelling blocks (its
    sum|w x| is 0), the others a deterministic mix of every kind."""
    cancel, other = kinds
    everything = cancel + other
    nb = k // 256
    g = np.random.default_rng(seed)
    rows = []
    for r in range(n):
        pool = cancel if r % 3 == 0 else everything
        idx = (g.integers(0, len(pool)) + np.arange(nb)) % len(pool)
        rows.append(np.concatenate([pool[i] for i in idx]))
    return np.stack(rows)


# ------------------------------------------------------------------ Q4_K GEMV

# Batch 1 (the decode kernel at one and two K steps, any row count), the FMA
# passes (2..4) and the split-bf16 MFMA kernel (5..32 rows, one and two batch
# tiles; 64-row weight tiles staged through LDS from 8192 rows).
@pytest.mark.parametrize("m,n,k", [(1, 200, 1024), (1, 8200, 512), (1, 8195, 4352),
                                   (2, 150, 768), (3, 97, 1024), (4, 64, 2304),
                                   (5, 130, 1024), (8, 8200, 256), (16, 77, 768),
                                   (17, 64, 512), (32, 300, 1280), (12, 8256, 1280),
                                   (30, 8200, 768)])
def test_q4k_gemv_structured(q4k, m, n, k):
    w = tile(q4k_kinds(), n, k, seed=m + n)
    x = synth.normal_f32((m, k), seed=m + k)
    y = q4k.gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.gemv(w, x, n, k)
    assert (a[:, ::3] == 0).all()
    assert_within(y, yr, a, GEMV_TOL, "q4k_gemv m=%d %dx%d" % (m, n, k))


def test_q4k_gemv_fully_cancelling_block_gives_zero(q4k):
    # d = dmin = 1, sc = 1, mn = 3, q = 3: every weight is 0, at every batch size
    k = 1024
    blk = pack_block(ONE, ONE, np.ones(8, int), np.full(8, 3), np.full(256, 3))
    w = np.tile(blk, (16, k // 256))
    wd = dev(w)
    for m in range(1, 33):
        x = synth.normal_f32((m, k), seed=m)
        y = q4k.gemv(wd, dev(x)).cpu().numpy()
        assert np.all(y == 0.0), "m=%d: %r" % (m, y[y != 0][:4])


# ------------------------------------------------------------------ Q5_K GEMV

@pytest.mark.parametrize("m,n,k", [(1, 200, 1024), (1, 8200, 512), (3, 64, 768), (5, 40, 512),
                                   (8, 130, 1024), (32, 64, 512)])
def test_q5k_gemv_structured(q4k, m, n, k):
    w = tile(q5k_kinds(), n, k, seed=m + n)
    x = synth.normal_f32((m, k), seed=m + k)
    y = q4k.q5k_gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.q5k_gemv(w, x, n, k)
    assert (a[:, ::3] == 0).all()
    assert_within(y, yr, a, GEMV_TOL, "q5k_gemv m=%d %dx%d" % (m, n, k))


# ------------------------------------------------------------------ Q6_K / Q3_K GEMV

@pytest.mark.parametrize("m,n,k", [(1, 100, 1024), (2, 33, 768), (4, 40, 4352), (6, 17, 512),
                                   (1, 8, 4352), (3, 40, 1280)])
def test_q6k_gemv_structured(q4k, m, n, k):
    w = tile(q6k_kinds(), n, k, seed=m + n)
    x = synth.normal_f32((m, k), seed=m + k)
    y = q4k.q6k_gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.q6k_gemv(w, x, n, k)
    assert (a[:, ::3] == 0).all()
    assert_within(y, yr, a, GEMV_TOL, "q6k_gemv m=%d %dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k", [(1, 100, 1024), (3, 40, 768), (5, 17, 4352), (1, 8, 4352),
                                   (2, 24, 8448)])
def test_q3k_gemv_structured(q4k, m, n, k):
    w = tile(q3k_kinds(), n, k, seed=m + n)
    x = synth.normal_f32((m, k), seed=m + k)
    y = q4k.q3k_gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.q3k_gemv(w, x, n, k)
    assert (a[:, ::3] == 0).all()
    assert_within(y, yr, a, GEMV_TOL, "q3k_gemv m=%d %dx%d" % (m, n, k))


# ------------------------------------------------------------------ GEMMs

# Split-K tiles, the streaming small-batch kernel (8, 16 and 32 staged X
# rows), the 64 x 64 / 64 x 128 K-slice tiles and the 128 x 256 tiles, all on
# structured weights.
@pytest.mark.parametrize("m,n,k", [(1, 130, 1024), (7, 8200, 256), (12, 8192, 1280),
                                   (30, 8256, 768), (40, 300, 768), (200, 6144, 256),
                                   (512, 4096, 512), (512, 8192, 256)])
def test_q4k_gemm_structured(q4k, m, n, k):
    w = tile(q4k_kinds(), n, k, seed=m + n)
    xb = synth.normal_bf16((m, k), seed=m + k)
    Y = q4k.gemm(dev(w), dev_bf16(xb)).cpu().numpy()
    cols = np.unique(np.concatenate([np.arange(0, min(n, 96)), [n - 2, n - 1],
                                     np.random.default_rng(n).integers(0, n, 64)]))
    Yr, A = oracle.gemm_cols(w, xb, n, k, cols)
    assert_within(Y[:, cols], Yr, A, GEMM_TOL, "q4k_gemm %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k", [(1, 130, 1024), (7, 8200, 256), (12, 8192, 1280),
                                   (30, 8256, 768), (40, 300, 768), (512, 4096, 512)])
def test_q5k_gemm_structured(q4k, m, n, k):
    w = tile(q5k_kinds(), n, k, seed=m + n)
    xb = synth.normal_bf16((m, k), seed=m + k)
    Y = q4k.q5k_gemm(dev(w), dev_bf16(xb)).cpu().numpy()
    cols = np.unique(np.concatenate([np.arange(0, min(n, 96)), [n - 1],
                                     np.random.default_rng(n).integers(0, n, 64)]))
    Yr, A = oracle.q5k_gemm_cols(w, xb, n, k, cols)
    assert_within(Y[:, cols], Yr, A, GEMM_TOL, "q5k_gemm %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("fmt,m,n,k", [("q6k", 1, 100, 1024), ("q6k", 64, 257, 768),
                                       ("q6k", 64, 264, 768), ("q3k", 1, 100, 1024),
                                       ("q3k", 64, 257, 768), ("q3k", 64, 264, 768)])
def test_plane_gemm_structured(q4k, fmt, m, n, k):
    kinds = q6k_kinds() if fmt == "q6k" else q3k_kinds()
    w = tile(kinds, n, k, seed=m + n)
    xb = synth.normal_bf16((m, k), seed=m + k)
    Y = getattr(q4k, fmt + "_gemm")(dev(w), dev_bf16(xb)).cpu().numpy()
    Yr, A = getattr(oracle, fmt + "_gemm")(w, xb, n, k)
    assert_within(Y, Yr, A, GEMM_TOL, "%s_gemm %dx%dx%d" % (fmt, m, n, k))


# ------------------------------------------------------------------ SwiGLU MLP

@pytest.mark.parametrize("dm,dff", [(512, 768), (1024, 2048)])
def test_swiglu_mlp_structured(q4k, dm, dff):
    kinds = q4k_kinds()
    # gate/up without the largest-finite kinds (their products overflow
    # silu's exp into its tails, which the seeded tests cover), down with all
    cancel, other = kinds
    mild = (cancel, [b for b in other if not (b[1] == 0x7B and b[0] == 0xFF)])
    wg = tile(mild, dff, dm, seed=1)
    wu = tile(mild, dff, dm, seed=2)
    wdn = tile(kinds, dm, dff, seed=3)
    x = synth.normal_f32(dm, seed=dm)
    out, h = q4k.swiglu_mlp(dev(wg), dev(wu), dev(wdn), dev(x))
    out = out.cpu().numpy()
    h = h.cpu().numpy()
    r = oracle.swiglu_mlp(wg, wu, wdn, x, dm, dff)
    g, u = r["g"], r["u"]
    silu = g / (1.0 + np.exp(-g))
    dg = GEMV_TOL * r["ag"]
    du = GEMV_TOL * r["au"]
    tol_h = 1.1 * np.abs(u) * dg + (np.abs(silu) + 1.1 * dg) * du + 1e-6 * np.abs(r["h"])
    err_h = np.abs(h.astype(np.float64) - r["h"])
    assert np.all(err_h <= tol_h), "h outside the propagated bound: worst %g at %d" % (
        (err_h - tol_h).max(), int(np.argmax(err_h - tol_h)))
    assert np.all(h[::3] == 0.0)  # gate rows that cancel: silu(0) * u = 0
    yd, ad = oracle.gemv(wdn, h, dm, dff)
    assert_within(out, yd[0], ad[0], GEMV_TOL, "mlp down stage")
    assert np.all(out[::3] == 0.0)  # down rows that cancel
