"""The torch binding refuses caller-supplied outputs of the wrong shape,
dtype or device before any kernel sees their pointers."""
from __future__ import annotations

import numpy as np
import pytest
import torch

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


def test_gemv_and_gemm_reject_missized_outputs(q4k):
    n, k = 64, 512
    w = torch.from_numpy(synth.q4k_weights(n, k, seed=1)).cuda()
    x = torch.zeros((3, k), dtype=torch.float32, device="cuda")
    for bad in (torch.empty((3, n - 1), device="cuda"), torch.empty((2, n), device="cuda"),
                torch.empty(3 * n, device="cuda"), torch.empty((3, n), device="cuda",
                                                                dtype=torch.float64)):
        with pytest.raises(ValueError):
            q4k.gemv(w, x, out=bad)
    with pytest.raises(ValueError):
        q4k.gemv(w, x[0], out=torch.empty(n - 1, device="cuda"))
    xb = torch.zeros((5, k), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        q4k.gemm(w, xb, out=torch.empty((5, n + 1), device="cuda"))
    y = torch.full((3, n), np.nan, device="cuda")
    assert q4k.gemv(w, x, out=y) is y and torch.all(y == 0)


def test_mlp_rejects_short_h_and_out(q4k):
    dm, dff = 256, 512
    wg = torch.from_numpy(synth.q4k_weights(dff, dm, seed=2)).cuda()
    wd = torch.from_numpy(synth.q4k_weights(dm, dff, seed=3)).cuda()
    x = torch.zeros(dm, device="cuda")
    with pytest.raises(ValueError):
        q4k.swiglu_mlp(wg, wg, wd, x, h=torch.empty(dff - 256, device="cuda"))
    with pytest.raises(ValueError):
        q4k.swiglu_mlp(wg, wg, wd, x, out=torch.empty(dm // 2, device="cuda"))
    with pytest.raises(ValueError):
        q4k.swiglu_mlp(wg, wg, wd, x.view(1, dm))


def test_w8a8_rejects_missized_output(q4k):
    x = torch.zeros((4, 128), dtype=torch.int8, device="cuda")
    w = torch.zeros((8, 128), dtype=torch.int8, device="cuda")
    s4 = torch.ones(4, device="cuda")
    s8 = torch.ones(8, device="cuda")
    with pytest.raises(ValueError):
        q4k.w8a8_linear(x, s4, w, s8, out=torch.empty((4, 7), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        q4k.w8a8_linear_acc(x, w, out=torch.empty((3, 8), dtype=torch.int32, device="cuda"))
