"""Q4_K, Q6_K and int8 weight matrices larger than 4 GiB through the GEMV and GEMM kernels.

The pages warn of 32-bit offsets on large tensors ("Writing an ESIMD Fused
Kernel From Reverse-Engineered Assembly", "The ABI Adapter and the int32
Overflow").  Here W has 1,900,000 rows of k = 4096 (4.38 GB): rows past the
4 GiB byte boundary (row 1,864,136 on) are checked against the oracle at
sampled columns, with the batch shapes that take each kernel family.  The
matrix is a 10,007-row seeded block (a prime period, so a row offset that
wrapped at 2^32 -- which lands mid-row -- cannot alias a correct row) tiled
on the device.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

N, K, PERIOD = 1_900_000, 4096, 10_007
ROW_BYTES = K // 256 * 144
FIRST_ROW_PAST_4G = (1 << 32) // ROW_BYTES + 1


@pytest.fixture(scope="module")
def big():
    if torch.cuda.device_count() == 0:
        pytest.skip("no GPU")
    import gemm_q4_super_block_amd as lib
    lib.load_library()
    torch.cuda.set_device(0)
    base = synth.q4k_weights(PERIOD, K, seed=11)
    wd = torch.empty((N, ROW_BYTES), dtype=torch.uint8, device="cuda")
    bd = torch.from_numpy(base).cuda()
    for r0 in range(0, N, PERIOD):
        r1 = min(N, r0 + PERIOD)
        wd[r0:r1].copy_(bd[: r1 - r0])
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, FIRST_ROW_PAST_4G - 1, FIRST_ROW_PAST_4G, N - 1],
                                     np.random.default_rng(5).integers(FIRST_ROW_PAST_4G, N, 12)]))
    yield lib, wd, base, rows
    del wd, bd
    torch.cuda.empty_cache()


def test_matrix_is_past_4gib(big):
    _, wd, _, _ = big
    assert wd.numel() > (1 << 32)
    assert FIRST_ROW_PAST_4G * ROW_BYTES >= (1 << 32) > (FIRST_ROW_PAST_4G - 1) * ROW_BYTES


@pytest.mark.parametrize("m", [1, 8])
def test_gemv_rows_past_4gib(big, m):
    lib, wd, base, rows = big
    x = synth.normal_f32((m, K), seed=m)
    y = lib.gemv(wd, torch.from_numpy(x).cuda()).cpu().numpy()
    yr, a = oracle.gemv_rows(base, x, PERIOD, K, rows % PERIOD)
    err = np.abs(y[:, rows] - yr)
    assert np.all(err <= 1e-4 * a), "worst %g" % (err / (1e-4 * a)).max()


@pytest.mark.parametrize("m", [8, 256])
def test_gemm_rows_past_4gib(big, m):
    lib, wd, base, rows = big
    xb = synth.normal_bf16((m, K), seed=m)
    xt = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    y = lib.gemm(wd, xt).cpu().numpy()
    yr, a = oracle.gemm_cols(base, xb, PERIOD, K, rows % PERIOD)
    err = np.abs(y[:, rows] - yr)
    assert np.all(err <= 1e-2 * a), "worst %g" % (err / (1e-2 * a)).max()


# ---- Q6_K (210-byte records) past 4 GiB: the plane GEMV and the plane GEMM whose operands
# are copied into LDS (the copies' 16-byte-aligned record spans, row pointers in 64 bits).
N6 = 1_300_000
ROW_BYTES_6 = K // 256 * 210
FIRST_ROW_PAST_4G_6 = (1 << 32) // ROW_BYTES_6 + 1


@pytest.fixture(scope="module")
def big6():
    if torch.cuda.device_count() == 0:
        pytest.skip("no GPU")
    import gemm_q4_super_block_amd as lib
    lib.load_library()
    torch.cuda.set_device(0)
    base = synth.q6k_weights(PERIOD, K, seed=12)
    wd = torch.empty((N6, ROW_BYTES_6), dtype=torch.uint8, device="cuda")
    bd = torch.from_numpy(base).cuda()
    for r0 in range(0, N6, PERIOD):
        r1 = min(N6, r0 + PERIOD)
        wd[r0:r1].copy_(bd[: r1 - r0])
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, FIRST_ROW_PAST_4G_6 - 1, FIRST_ROW_PAST_4G_6, N6 - 1],
                                     np.random.default_rng(6).integers(FIRST_ROW_PAST_4G_6, N6, 12)]))
    yield lib, wd, base, rows
    del wd, bd
    torch.cuda.empty_cache()


def test_q6k_matrix_is_past_4gib(big6):
    _, wd, _, _ = big6
    assert wd.numel() > (1 << 32)
    assert FIRST_ROW_PAST_4G_6 * ROW_BYTES_6 >= (1 << 32) > (FIRST_ROW_PAST_4G_6 - 1) * ROW_BYTES_6
    assert (N6 * (K // 256)) % 8 == 0  # the GEMM takes the LDS-staged kernel


def test_q6k_gemv_rows_past_4gib(big6):
    lib, wd, base, rows = big6
    x = synth.normal_f32((1, K), seed=21)
    y = lib.q6k_gemv(wd, torch.from_numpy(x).cuda()).cpu().numpy().reshape(1, -1)
    yr, a = oracle.q6k_gemv_rows(base, x, PERIOD, K, rows % PERIOD)
    err = np.abs(y[:, rows] - yr)
    assert np.all(err <= 1e-4 * a), "worst %g" % (err / (1e-4 * a)).max()


def test_q6k_gemm_rows_past_4gib(big6):
    lib, wd, base, rows = big6
    m = 64
    xb = synth.normal_bf16((m, K), seed=22)
    xt = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    y = lib.q6k_gemm(wd, xt).cpu().numpy()
    yr, a = oracle.q6k_gemm_cols(base, xb, PERIOD, K, rows % PERIOD)
    err = np.abs(y[:, rows] - yr)
    assert np.all(err <= 1e-2 * a), "worst %g" % (err / (1e-2 * a)).max()


# ---- INT8 W8A8 weights past 4 GiB (int8 [n, k], the 128 x 192 tiles), bit for bit.
N8 = 1_105_920  # a multiple of 128 and of 192
FIRST_ROW_PAST_4G_8 = (1 << 32) // K + 1


def test_w8a8_rows_past_4gib():
    if torch.cuda.device_count() == 0:
        pytest.skip("no GPU")
    import gemm_q4_super_block_amd as lib
    lib.load_library()
    torch.cuda.set_device(0)
    m = 64
    x, xs, w, ws, b = synth.w8a8_case(m, PERIOD, K, seed=13)
    wd = torch.empty((N8, K), dtype=torch.int8, device="cuda")
    bd = torch.from_numpy(w).cuda()
    for r0 in range(0, N8, PERIOD):
        r1 = min(N8, r0 + PERIOD)
        wd[r0:r1].copy_(bd[: r1 - r0])
    assert wd.numel() > (1 << 32)
    wsd = torch.from_numpy(np.resize(ws, N8)).cuda()
    b_d = torch.from_numpy(np.resize(b, N8)).cuda()
    y = lib.w8a8_linear(torch.from_numpy(x).cuda(), torch.from_numpy(xs).cuda(), wd, wsd, b_d)
    rows = np.unique(np.concatenate([[0, FIRST_ROW_PAST_4G_8 - 1, FIRST_ROW_PAST_4G_8, N8 - 1],
                                     np.random.default_rng(8).integers(FIRST_ROW_PAST_4G_8, N8, 12)]))
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)[:, rows]
    ref = oracle.w8a8_linear_cols(x, xs, w, ws, b, rows % PERIOD)
    del wd, bd, wsd, b_d, y
    torch.cuda.empty_cache()
    assert np.array_equal(got, ref), "%d of %d outputs differ" % ((got != ref).sum(), got.size)
