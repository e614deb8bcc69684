"""q4k_swiglu_mlp_noalloc (h in the library's static device scratch) against
q4k_swiglu_mlp (h a caller buffer), through the C ABI.

The two entry points run the same kernels, so their outputs must agree bit
for bit; the no-allocation call is checked on two calls in a row, the second
on a smaller MLP (its scratch then still holds the first call's longer h).
The allocating call's own h is checked against the oracle's down stage.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if torch.cuda.device_count() == 0:
        pytest.skip("no GPU")
    from gemm_q4_super_block_amd import _lib
    _lib.load()
    torch.cuda.set_device(0)
    return _lib


def _case(dm, dff, seed):
    wg = synth.q4k_weights(dff, dm, seed=seed, stream=synth.W_GATE)
    wu = synth.q4k_weights(dff, dm, seed=seed, stream=synth.W_UP)
    wd = synth.q4k_weights(dm, dff, seed=seed, stream=synth.W_DOWN)
    x = synth.normal_f32(dm, seed=seed)
    return wd, [torch.from_numpy(a).cuda() for a in (wg, wu, wd, x)]


def test_noalloc_matches_the_allocating_entry_point(lib):
    stream = torch.cuda.current_stream().cuda_stream
    for dm, dff, seed in ((4096, 14336, 0), (512, 1024, 1)):  # second call smaller
        wd_host, (g, u, d, x) = _case(dm, dff, seed)
        h = torch.full((dff,), float("nan"), device="cuda")
        ref = torch.full((dm,), float("nan"), device="cuda")
        out = torch.full((dm,), float("nan"), device="cuda")
        assert lib.q4k_swiglu_mlp(g.data_ptr(), u.data_ptr(), d.data_ptr(), x.data_ptr(),
                                  h.data_ptr(), ref.data_ptr(), dm, dff, stream) == lib.Q4K_OK
        assert lib.q4k_swiglu_mlp_noalloc(g.data_ptr(), u.data_ptr(), d.data_ptr(), x.data_ptr(),
                                          out.data_ptr(), dm, dff, stream) == lib.Q4K_OK
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        r = ref.cpu().numpy()
        assert np.array_equal(o.view(np.uint32), r.view(np.uint32)), (dm, dff)
        yd, ad = oracle.gemv(wd_host, h.cpu().numpy(), dm, dff)
        assert np.all(np.abs(o.astype(np.float64) - yd[0]) <= 1e-4 * ad[0]), (dm, dff)


def test_noalloc_rejects_d_ff_past_its_scratch(lib):
    A = 1 << 20  # never dereferenced: the size check fails first
    too_big = lib.Q4K_NOALLOC_MAX_D_FF + 256
    rc = lib.q4k_swiglu_mlp_noalloc(A, 2 * A, 3 * A, 4 * A, 5 * A, 4096, too_big, None)
    assert rc == lib.Q4K_ERR_INVALID_ARG
    assert "Q4K_NOALLOC_MAX_D_FF" in lib.q4k_last_error()
