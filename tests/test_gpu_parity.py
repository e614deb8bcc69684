"""Parity of the HIP path (libq4k through its C ABI) with the CPU oracle.

Every test here runs on an MI355X and compares the GPU result element by
element with the oracle on the same seeded inputs:
  * dequantized weights: bit-exact (fp32, and bf16 = nearest-even of fp32);
  * fp32 GEMV / sweep GEMV: |y - y_oracle| <= 1e-4 * sum|w x| per output;
  * bf16-MFMA GEMM: |Y - Y_oracle| <= 1e-2 * sum|w x| per output;
  * SwiGLU MLP: h within the first-order propagation of the GEMV tolerance
    through silu(g)*u, the down projection within 1e-4 * sum|w_down h| of the
    oracle run on the GPU's own h, and the end-to-end output within the sum
    of both.
Shapes cover the five workload configurations (at full size, on sampled
outputs where the oracle would be slow), tiles plus ragged tails, and the
degenerate cases of the format (subnormal scales, zero and maximal fields).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from golden_io import hand_blocks
from q4k_pack import pack_block

pytestmark = pytest.mark.gpu

GEMV_TOL = 1e-4
GEMM_TOL = 1e-2


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
        raise AssertionError("%s: %d outputs outside %g * sum|w x|; worst at %s: got %r ref %r "
                             "bound %r" % (what, bad.sum(), tol, np.unravel_index(i, err.shape),
                                           got.flat[i], ref.flat[i], bound.flat[i]))
    return float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0


# ------------------------------------------------------------------ dequant

@pytest.mark.parametrize("n,k,seed", [(256, 1024, 0), (256, 1024, 1), (256, 1024, 2),
                                      (4096, 4096, 0), (7, 14336, 3)])
def test_dequant_bit_exact(q4k, n, k, seed):
    w = synth.q4k_weights(n, k, seed=seed)
    wd = dev(w)
    got32 = q4k.dequantize_f32(wd).cpu().numpy()
    ref32 = oracle.dequant_f32(w, n, k)
    assert np.array_equal(got32.view(np.uint32), ref32.view(np.uint32))
    got16 = q4k.dequantize_bf16(wd).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got16, oracle.dequant_bf16(w, n, k))


def test_dequant_hand_packed_blocks(q4k):
    blocks = hand_blocks()
    names = sorted(blocks)
    w = np.stack([blocks[nm][0] for nm in names])          # [5, 144]: one block per row
    got = q4k.dequantize_f32(dev(w)).cpu().numpy().astype(np.float64)
    for i, nm in enumerate(names):
        assert np.array_equal(got[i], blocks[nm][1]), nm


def test_dequant_degenerate_fields(q4k):
    g = np.random.default_rng(99)
    rows = []
    # subnormal d and dmin, every combination of extreme scales, zero and 15 quants
    for d in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF):
        for dmin in (0x0000, 0x0001, 0x0200, 0x3C00):
            sc = g.integers(0, 64, 8)
            mn = g.integers(0, 64, 8)
            sc[0], mn[0], sc[7], mn[7] = 63, 63, 0, 0
            q = g.integers(0, 16, 256)
            q[:32] = 15
            q[32:64] = 0
            rows.append(pack_block(d, dmin, sc, mn, q))
    w = np.stack(rows)
    n, k = w.shape[0], 256
    got = q4k.dequantize_f32(dev(w)).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oracle.dequant_f32(w, n, k).view(np.uint32))
    got16 = q4k.dequantize_bf16(dev(w)).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got16, oracle.dequant_bf16(w, n, k))


# ------------------------------------------------------------------ GEMV

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gemv_config_small(q4k, seed):
    # 256 x 1024 (4 super-blocks per row), batch 1
    n, k = 256, 1024
    w = synth.q4k_weights(n, k, seed=seed)
    x = synth.normal_f32(k, seed=seed)
    y = q4k.gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.gemv(w, x, n, k)
    assert_within(y, yr[0], a[0], GEMV_TOL, "gemv 256x1024 seed %d" % seed)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gemv_decode_4096(q4k, seed):
    n = k = 4096
    w = synth.q4k_weights(n, k, seed=seed)
    x = synth.normal_f32(k, seed=seed)
    y = q4k.gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.gemv(w, x, n, k)
    assert_within(y, yr[0], a[0], GEMV_TOL, "gemv 4096x4096 seed %d" % seed)


# Batch 1 at k <= 16384 runs the decode kernel (8 rows per workgroup; one to
# four K steps of 4096, ragged last steps of one block (8448) and of 49 blocks
# (12544), the largest k, rows not a multiple of 8, tall matrices: 8200 x 768
# leaves 13 of the 16 super-block lanes idle).  The general kernel's batch-1
# shapes are covered through Q5_K, which runs them at every size.
@pytest.mark.parametrize("n,k", [(1, 256), (17, 256), (257, 768), (100, 3840), (33, 4352),
                                 (64, 14336), (1000, 1280), (50, 8448), (5, 9216), (7, 12544),
                                 (4100, 16384), (8192, 2304), (8200, 768), (9001, 4096),
                                 (8193, 4352)])
def test_gemv_ragged_shapes(q4k, n, k):
    w = synth.q4k_weights(n, k, seed=5)
    x = synth.normal_f32(k, seed=5)
    y = q4k.gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.gemv(w, x, n, k)
    assert_within(y, yr[0], a[0], GEMV_TOL, "gemv %dx%d" % (n, k))


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 7, 8, 9, 16, 31, 32])
def test_gemv_batched(q4k, m):
    n, k = 300, 1024
    w = synth.q4k_weights(n, k, seed=m)
    x = synth.normal_f32((m, k), seed=m)
    y = q4k.gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.gemv(w, x, n, k)
    assert_within(y, yr, a, GEMV_TOL, "gemv m=%d" % m)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("m", [1, 2, 4, 8, 16, 32])
def test_gemv_sweep_shape_sampled(q4k, m, seed):
    # 14336 x 4096 weights, fp32 X [m, 4096]; oracle on sampled output rows
    n, k = 14336, 4096
    w = synth.q4k_weights(n, k, seed=seed)
    x = synth.normal_f32((m, k), seed=seed)
    y = q4k.gemv(dev(w), dev(x)).cpu().numpy()
    rows = np.unique(np.concatenate([[0, 1, n - 1, n - 2],
                                     np.random.default_rng(m + seed).integers(0, n, 96)]))
    yr, a = oracle.gemv_rows(w, x, n, k, rows)
    assert_within(y[:, rows], yr, a, GEMV_TOL, "sweep gemv m=%d seed %d" % (m, seed))


def test_gemv_unit_vectors_give_columns(q4k):
    # y(e_c) is column c of the dequantized W, exactly (one non-zero product)
    n, k = 40, 512
    w = synth.q4k_weights(n, k, seed=21)
    W = oracle.dequant_f32(w, n, k)
    wd = dev(w)
    for c in (0, 1, 31, 32, 63, 64, 100, 255, 256, 300, 511):
        x = np.zeros(k, np.float32)
        x[c] = 1.0
        y = q4k.gemv(wd, dev(x)).cpu().numpy()
        assert np.array_equal(y, W[:, c]), c


def test_gemv_split_unit_vectors_within_weight_split(q4k):
    # Batches of 5..32 rows take the split-bf16 MFMA kernel: for x = e_c the
    # output is w_hi + w_lo of each weight of column c, within 2^-16 |w|
    # (and exactly 0 where the weight is 0).
    n, k = 40, 512
    w = synth.q4k_weights(n, k, seed=22)
    W = oracle.dequant_f32(w, n, k).astype(np.float64)
    cols = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 300, 511]
    x = np.zeros((len(cols), k), np.float32)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    y = q4k.gemv(dev(w), dev(x)).cpu().numpy()
    for i, c in enumerate(cols):
        assert np.all(np.abs(y[i] - W[:, c]) <= 2.0 ** -16 * np.abs(W[:, c])), c


# ------------------------------------------------------------------ SwiGLU MLP

def _mlp_check(q4k, dm, dff, seed, x_scale=1.0):
    wg = synth.q4k_weights(dff, dm, seed=seed, stream=synth.W_GATE)
    wu = synth.q4k_weights(dff, dm, seed=seed, stream=synth.W_UP)
    wdn = synth.q4k_weights(dm, dff, seed=seed, stream=synth.W_DOWN)
    x = synth.normal_f32(dm, seed=seed) * np.float32(x_scale)
    out, h = q4k.swiglu_mlp(dev(wg), dev(wu), dev(wdn), dev(x))
    out = out.cpu().numpy()
    h = h.cpu().numpy()
    r = oracle.swiglu_mlp(wg, wu, wdn, x, dm, dff)
    g, u = r["g"], r["u"]
    sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dg = GEMV_TOL * r["ag"]
    du = GEMV_TOL * r["au"]
    # |silu'| <= 1.1 everywhere; first-order propagation plus fp32 rounding of h
    tol_h = 1.1 * np.abs(u) * dg + (np.abs(silu) + 1.1 * dg) * du + 1e-6 * np.abs(r["h"]) + 1e-30
    err_h = np.abs(h.astype(np.float64) - r["h"])
    assert np.all(err_h <= tol_h), "h outside propagated bound (worst ratio %g)" % (
        (err_h / tol_h).max())
    # down stage on the GPU's own h
    yd, ad = oracle.gemv(wdn, h, dm, dff)
    assert_within(out, yd[0], ad[0], GEMV_TOL, "mlp down stage")
    # end to end: down-stage tolerance plus the propagated h tolerance
    D = np.abs(oracle.dequant_f32(wdn, dm, dff))
    prop = (D @ tol_h.astype(np.float32)).astype(np.float64) * 1.01
    err = np.abs(out - r["out"])
    assert np.all(err <= GEMV_TOL * r["aout"] * 1.01 + prop), "mlp end to end"


# d_model of one to four K steps of 4096 (ragged: 4352, 8448, 12544).
@pytest.mark.parametrize("dm,dff,seed", [(256, 512, 0), (512, 768, 1), (1024, 3840, 2),
                                         (4352, 512, 3), (8448, 256, 4), (12544, 768, 5),
                                         (16384, 256, 6)])
def test_swiglu_mlp_small(q4k, dm, dff, seed):
    _mlp_check(q4k, dm, dff, seed)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_swiglu_mlp_llama_shape(q4k, seed):
    # d_model 4096, d_ff 14336 (the decode MLP configuration), full oracle
    _mlp_check(q4k, 4096, 14336, seed)


def test_swiglu_mlp_large_activations(q4k):
    # pre-activations far into both silu tails
    _mlp_check(q4k, 512, 1024, 3, x_scale=50.0)


# ------------------------------------------------------------------ GEMM

@pytest.mark.parametrize("m,n,k", [(1, 128, 256), (9, 300, 512), (31, 128, 1024), (32, 256, 768),
                                   (33, 130, 512), (100, 384, 1024), (256, 128, 256),
                                   (257, 260, 768), (512, 256, 1280)])
def test_gemm_small_shapes(q4k, m, n, k):
    w = synth.q4k_weights(n, k, seed=m)
    xb = synth.normal_bf16((m, k), seed=m)
    Y = q4k.gemm(dev(w), dev_bf16(xb)).cpu().numpy()
    Yr, A = oracle.gemm(w, xb, n, k)
    assert_within(Y, Yr, A, GEMM_TOL, "gemm %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("n", [4096, 14336])
def test_gemm_prefill_sampled(q4k, n, seed):
    # X bf16 [512, 4096], W [n, 4096]: all 512 rows at 64 sampled columns
    m, k = 512, 4096
    w = synth.q4k_weights(n, k, seed=seed)
    xb = synth.normal_bf16((m, k), seed=seed)
    Y = q4k.gemm(dev(w), dev_bf16(xb)).cpu().numpy()
    cols = np.unique(np.concatenate([[0, 1, 127, 128, n - 1],
                                     np.random.default_rng(n + seed).integers(0, n, 59)]))
    Yr, A = oracle.gemm_cols(w, xb, n, k, cols)
    assert_within(Y[:, cols], Yr, A, GEMM_TOL, "gemm 512x%dx4096 seed %d" % (n, seed))
    assert np.all(np.isfinite(Y))


# Shapes around the kernel switches (M > 32):
#   128 x 256 tiles (M >= 256, >= 128 tiles): an XCD-ordered grid of exactly 128
#     tiles at the smallest K (one super-block); ragged M and N, 192 tiles, three
#     super-blocks (every K rotation in play); ragged M with the linear order;
#     five M-tiles on the XCD order.
#   64 x 128 tiles (>= 192 tiles): ragged M and N (325 tiles), N not a multiple
#     of 128 with 192 tiles, M = 65 (a one-row last M-tile), 256 tiles at K = 4096.
#   64 x 64 tiles (fewer than 192 of 64 x 128, >= 192 of 64 x 64): 256 tiles,
#     ragged N with 196 tiles, a one-row last M-tile with 282 tiles.
#   128 x 128 tiles with split K (fewer tiles): 64 and 32 tiles.
@pytest.mark.parametrize("m,n,k", [(512, 8192, 256), (257, 16383, 768), (300, 16640, 512),
                                   (640, 12288, 1024), (300, 8200, 512), (384, 4000, 4096),
                                   (65, 24576, 512), (512, 4096, 4096), (256, 4096, 512),
                                   (200, 3100, 768), (129, 6000, 256), (128, 4096, 1024),
                                   (64, 4000, 2048)])
def test_gemm_tile_kernels(q4k, m, n, k):
    w = synth.q4k_weights(n, k, seed=m + k)
    xb = synth.normal_bf16((m, k), seed=m + k)
    Y = q4k.gemm(dev(w), dev_bf16(xb)).cpu().numpy()
    cols = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 255, 256, n - 129, n - 65, n - 2,
                                      n - 1], np.random.default_rng(n).integers(0, n, 52)]))
    Yr, A = oracle.gemm_cols(w, xb, n, k, cols)
    assert_within(Y[:, cols], Yr, A, GEMM_TOL, "gemm %dx%dx%d" % (m, n, k))
    assert np.all(np.isfinite(Y))


# Batches of at most 32 rows with >= 128 weight tiles of 64 rows run the
# streaming kernel: X staged for 8 rows (m <= 8), 16 rows (m <= 16) or 32, with
# 32- or 64-row weight tiles; each wave of a workgroup takes every fourth
# super-block, so K of 1, 3, 5, 9 and 17 super-blocks leaves waves idle or with
# odd counts.  Ragged N (8200: an 8-row last tile) and the batch sizes at each
# staging switch.
@pytest.mark.parametrize("m,n,k", [(1, 8200, 256), (5, 8200, 256), (8, 8224, 1280),
                                   (9, 9000, 768), (16, 8192, 2304), (17, 9000, 768),
                                   (32, 16384, 512), (32, 8200, 4352)])
def test_gemm_small_batch_stream(q4k, m, n, k):
    w = synth.q4k_weights(n, k, seed=m + n)
    xb = synth.normal_bf16((m, k), seed=m + n)
    Y = q4k.gemm(dev(w), dev_bf16(xb)).cpu().numpy()
    cols = np.unique(np.concatenate([[0, 1, 31, 32, 63, 64, n - 65, n - 64, n - 33, n - 32,
                                      n - 9, n - 1], np.random.default_rng(n).integers(0, n, 52)]))
    Yr, A = oracle.gemm_cols(w, xb, n, k, cols)
    assert_within(Y[:, cols], Yr, A, GEMM_TOL, "gemm %dx%dx%d" % (m, n, k))
    assert np.all(np.isfinite(Y))


@pytest.mark.parametrize("m,n,k", [(7, 8192, 256), (13, 8192, 1024)])
def test_gemm_small_batch_stream_full_output(q4k, m, n, k):
    w = synth.q4k_weights(n, k, seed=78 + m)
    xb = synth.normal_bf16((m, k), seed=78 + m)
    Y = q4k.gemm(dev(w), dev_bf16(xb)).cpu().numpy()
    Yr, A = oracle.gemm(w, xb, n, k)
    assert_within(Y, Yr, A, GEMM_TOL, "gemm %dx%dx%d" % (m, n, k))


def test_gemm_mid_tile_kernel_full_output(q4k):
    # 4 x 48 = 192 tiles of 64 x 128 (the smallest mid-tile grid), every output
    # against the oracle; M = 200 leaves an 8-row last M-tile.
    m, n, k = 200, 6144, 256
    w = synth.q4k_weights(n, k, seed=77)
    xb = synth.normal_bf16((m, k), seed=77)
    Y = q4k.gemm(dev(w), dev_bf16(xb)).cpu().numpy()
    Yr, A = oracle.gemm(w, xb, n, k)
    assert_within(Y, Yr, A, GEMM_TOL, "gemm 200x6144x256")


# Every output of the two grids whose tiles are dealt to the XCDs in 2 x 4
# blocks (M split in two): 6 x 32 tiles of 64 x 128 and 4 x 36 tiles of
# 128 x 256 (N = 9216 is not a multiple of eight 256-column tiles per XCD).
@pytest.mark.parametrize("m,n,k", [(384, 4096, 256), (512, 9216, 256)])
def test_gemm_xcd_blocked_grids_full_output(q4k, m, n, k):
    w = synth.q4k_weights(n, k, seed=n + 5)
    xb = synth.normal_bf16((m, k), seed=n + 5)
    Y = q4k.gemm(dev(w), dev_bf16(xb)).cpu().numpy()
    Yr, A = oracle.gemm(w, xb, n, k)
    assert_within(Y, Yr, A, GEMM_TOL, "gemm %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("m", [1, 2, 4, 8, 16, 32])
def test_gemm_sweep_shape_sampled(q4k, m, seed):
    n, k = 14336, 4096
    w = synth.q4k_weights(n, k, seed=seed)
    xb = synth.bf16_bits(synth.normal_f32((m, k), seed=seed))
    Y = q4k.gemm(dev(w), dev_bf16(xb)).cpu().numpy()
    cols = np.unique(np.concatenate([[0, n - 1],
                                     np.random.default_rng(m + seed).integers(0, n, 62)]))
    Yr, A = oracle.gemm_cols(w, xb, n, k, cols)
    assert_within(Y[:, cols], Yr, A, GEMM_TOL, "sweep gemm m=%d seed %d" % (m, seed))


def test_gemm_m1_equals_bf16_weight_dot(q4k):
    # With X exactly representable, the GEMM at m=1 is the dot of X with the
    # bf16 weights the GPU exports; compare with that (tighter than 1e-2)
    n, k = 256, 2048
    w = synth.q4k_weights(n, k, seed=30)
    xb = synth.normal_bf16((1, k), seed=30)
    Y = q4k.gemm(dev(w), dev_bf16(xb)).cpu().numpy().astype(np.float64)
    Wb = oracle.dequant_bf16(w, n, k)
    Wf = (Wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = Xf @ Wf.T
    scale = np.abs(Xf) @ np.abs(Wf.T)
    assert np.all(np.abs(Y - ref) <= 1e-5 * scale)


# ------------------------------------------------------------------ read probe

@pytest.mark.parametrize("nbytes", [16, 144 * 4096, 9437184 + 48])
def test_read_probe_runs_and_leaves_sink(q4k, nbytes):
    """The streaming read probe (a measurement aid) reads the whole buffer and, for data
    whose folded sum is not its sentinel value, leaves the sink untouched."""
    from gemm_q4_super_block_amd import _lib
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    assert _lib.q4k_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(),
                               torch.cuda.current_stream().cuda_stream) == _lib.Q4K_OK
    torch.cuda.synchronize()
    assert sink.cpu().tolist() == [7, 7, 7, 7]


# ------------------------------------------------------------------ K chunks

# x is staged a chunk of K at a time (16384 elements at batch 1, 8192 at
# batch 2, 4096 for larger batches); past one chunk each chunk's partial dot
# is added into y.  Batch 1 below and above 8192 rows, batch 2 over two
# chunks, a batch of 3 over two and a batch of 8 over three.
@pytest.mark.parametrize("m,n,k", [(1, 300, 20480), (1, 9000, 16640), (2, 257, 9216),
                                   (3, 130, 4352), (8, 64, 8448)])
def test_gemv_multi_chunk_k(q4k, m, n, k):
    w = synth.q4k_weights(n, k, seed=k + m)
    x = synth.normal_f32((m, k), seed=k + m)
    y = q4k.gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.gemv(w, x, n, k)
    assert_within(y, yr, a, GEMV_TOL, "gemv m=%d %dx%d" % (m, n, k))


def test_swiglu_mlp_d_model_past_one_chunk(q4k):
    # d_model > 16384: the gate/up pair keeps one row set per wave so its two
    # dots stay in registers across x chunks until silu.
    dm, dff = 16640, 512
    _mlp_check(q4k, dm, dff, 7)


def test_gemm_long_k(q4k):
    m, n, k = 64, 512, 16384
    w = synth.q4k_weights(n, k, seed=3)
    xb = synth.normal_bf16((m, k), seed=3)
    Y = q4k.gemm(dev(w), dev_bf16(xb)).cpu().numpy()
    cols = np.arange(0, n, 7)
    Yr, A = oracle.gemm_cols(w, xb, n, k, cols)
    assert_within(Y[:, cols], Yr, A, GEMM_TOL, "gemm 64x512x16384")


# ------------------------------------------------------------------ split-bf16 MFMA GEMV

# Q4_K batches of 5..32 rows run on bf16 MFMA with the exact fp32 weights and
# x each split into bf16 hi + lo (three MFMAs per tile).  Edges: one
# super-block (only the first of the four K-split waves has work), a block
# count not divisible by four, single and ragged 16-row weight tiles, batch
# sizes around the 16-row MFMA tile, matrices past 8192 rows (64-row
# weight tiles staged through LDS: ragged rows, fewer super-blocks than the
# eight K-split waves, a block count not divisible by eight, one and two
# batch tiles), and x spanning six decades.
@pytest.mark.parametrize("m,n,k", [(5, 1, 256), (6, 1, 256), (15, 17, 256), (16, 33, 1280),
                                   (17, 16, 4352), (32, 15, 768), (7, 4096, 4096),
                                   (24, 500, 2048), (5, 8200, 512), (20, 8192, 256),
                                   (8, 8250, 1280), (12, 16384, 2048), (32, 9000, 4352)])
def test_gemv_split_edges(q4k, m, n, k):
    w = synth.q4k_weights(n, k, seed=m + n)
    x = synth.normal_f32((m, k), seed=m + n)
    y = q4k.gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.gemv(w, x, n, k)
    assert_within(y, yr, a, GEMV_TOL, "split gemv m=%d %dx%d" % (m, n, k))


def test_gemv_split_wide_dynamic_range(q4k):
    m, n, k = 8, 64, 1024
    w = synth.q4k_weights(n, k, seed=77)
    g = synth.rng(77, synth.X)
    x = (synth.normal_f32((m, k), seed=77) * 10.0 ** g.uniform(-3, 3, (m, k))).astype(np.float32)
    y = q4k.gemv(dev(w), dev(x)).cpu().numpy()
    yr, a = oracle.gemv(w, x, n, k)
    assert_within(y, yr, a, GEMV_TOL, "split gemv, x over six decades")
