"""q4k_gemv_layers: independent decode GEMVs of one shape in one persistent launch.

Every layer's output is checked against the oracle's GEMV of that layer at the
GEMV bar (1e-4 * sum|w x| per output), for layer counts from 1 to the maximum,
shared and distinct x, one or several rows per wave and layer, waves without
rows, several K steps, and layers built from structured and cancelling blocks
(whose rows must come out +-0); and bit for bit against q4k_gemv.
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


def _check(q4k, ws, xs, n, k, what):
    ys = q4k.gemv_layers([torch.from_numpy(w).cuda() for w in ws],
                         [torch.from_numpy(x).cuda() for x in xs])
    for l, (w, x, y) in enumerate(zip(ws, xs, ys)):
        yr, a = oracle.gemv(w, x, n, k)
        err = np.abs(y.cpu().numpy().astype(np.float64) - yr[0])
        assert np.all(err <= 1e-4 * a[0]), "%s layer %d: worst %g" % (
            what, l, (err / np.maximum(1e-4 * a[0], 1e-300)).max())


# One row per wave per layer (4096 rows), several (8200, 8195 rows: 256
# workgroups of 16 waves), waves with no rows (50 rows at the largest k),
# K steps past the first with a ragged last one (12544 = 49 super-blocks),
# every layer count from 1 to the maximum.
@pytest.mark.parametrize("layers,n,k,shared", [(1, 4096, 4096, False), (8, 4096, 4096, False),
                                               (3, 300, 1024, True), (32, 256, 256, False),
                                               (2, 8200, 512, False), (2, 8195, 4352, True),
                                               (3, 50, 16384, False), (4, 130, 12544, True)])
def test_layers_match_the_oracle(q4k, layers, n, k, shared):
    ws = [synth.q4k_weights(n, k, seed=100 + l) for l in range(layers)]
    xs = [synth.normal_f32(k, seed=0 if shared else 200 + l) for l in range(layers)]
    _check(q4k, ws, xs, n, k, "%d layers %dx%d" % (layers, n, k))


@pytest.mark.parametrize("n,k", [(1000, 1280), (257, 9216), (300, 14336)])
def test_layers_equal_separate_gemvs(q4k, n, k):
    # the same per-row arithmetic as q4k_gemv (one to four K steps): bit-identical outputs
    layers = 5
    ws = [torch.from_numpy(synth.q4k_weights(n, k, seed=300 + l)).cuda() for l in range(layers)]
    xs = [torch.from_numpy(synth.normal_f32(k, seed=400 + l)).cuda() for l in range(layers)]
    ys = q4k.gemv_layers(ws, xs)
    for w, x, y in zip(ws, xs, ys):
        ref = q4k.gemv(w, x)
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32))


def test_layers_structured_blocks(q4k):
    from test_gpu_structured import q4k_kinds, tile
    n, k, layers = 90, 768, 4
    ws = [tile(q4k_kinds(), n, k, seed=l) for l in range(layers)]
    xs = [synth.normal_f32(k, seed=500 + l) for l in range(layers)]
    _check(q4k, ws, xs, n, k, "structured layers")
    ys = q4k.gemv_layers([torch.from_numpy(w).cuda() for w in ws],
                         [torch.from_numpy(x).cuda() for x in xs])
    for y in ys:
        assert torch.all(y[::3] == 0)
