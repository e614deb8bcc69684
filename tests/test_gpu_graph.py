"""The HIP path under HIP graph capture (torch.cuda.graph).

Every entry point enqueues kernels only (no memset nodes, no allocation, no
host synchronization), so a captured sequence must replay to the eager
results.  The sequence covers every kernel family: batch-1 and batched GEMV,
the GEMM kernels (128 x 256, 64 x 128 K-slice, the streaming kernel for
small batches at each X staging size, split K with its zeroing kernel), the SwiGLU MLP (also without allocation), the layered
GEMV and the dequant export.  Between replays
the outputs are overwritten eagerly with NaN, and every replay is compared
with the eager run: bit for bit where the kernel's summation order is fixed,
and within the oracle tolerance where split K adds partial tiles with fp32
atomics (order not fixed).
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


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


# (m, n, k, exact): GEMM shapes per kernel family
GEMMS = [(512, 8192, 256, True),    # 128 x 256 tiles (4 x 32 = 128)
         (384, 4096, 256, True),    # 64 x 128 K-slice (6 x 32 = 192)
         (8, 8192, 256, True),      # streaming, X staged for 8 rows
         (16, 8192, 768, True),     # streaming, 16 rows
         (32, 8192, 1024, True),    # streaming, 32 rows, 64-row weight tiles
         (64, 4000, 2048, False),   # split K over 128 x 128 tiles
         (5, 1000, 1024, False)]    # small batch, split K


def test_graph_replays_match_eager(q4k):
    ops = []  # (name, run(), outputs, exact)
    # GEMV: batch 1 and a batch of 3
    for m in (1, 3):
        n, k = 2048, 1024
        w = dev(synth.q4k_weights(n, k, seed=40 + m))
        x = dev(synth.normal_f32((m, k), seed=40 + m))
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        ops.append(("gemv m=%d" % m, lambda w=w, x=x, y=y: q4k.gemv(w, x, out=y), [y], True))
    for m, n, k, exact in GEMMS:
        w = dev(synth.q4k_weights(n, k, seed=m + n))
        xb = dev_bf16(synth.normal_bf16((m, k), seed=m + n))
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        ops.append(("gemm %dx%dx%d" % (m, n, k), lambda w=w, xb=xb, y=y: q4k.gemm(w, xb, out=y),
                    [y], exact))
    dm, dff = 1024, 2048
    wg = dev(synth.q4k_weights(dff, dm, seed=1, stream=synth.W_GATE))
    wu = dev(synth.q4k_weights(dff, dm, seed=1, stream=synth.W_UP))
    wd = dev(synth.q4k_weights(dm, dff, seed=1, stream=synth.W_DOWN))
    xm = dev(synth.normal_f32(dm, seed=1))
    h = torch.empty(dff, dtype=torch.float32, device="cuda")
    o = torch.empty(dm, dtype=torch.float32, device="cuda")
    ops.append(("mlp", lambda: q4k.swiglu_mlp(wg, wu, wd, xm, h=h, out=o), [h, o], True))
    o2 = torch.empty(dm, dtype=torch.float32, device="cuda")
    ops.append(("mlp without allocation", lambda: q4k.swiglu_mlp_noalloc(wg, wu, wd, xm, o2),
                [o2], True))
    lw = [dev(synth.q4k_weights(1024, 512, seed=60 + l)) for l in range(3)]
    lx = [dev(synth.normal_f32(512, seed=60 + l)) for l in range(3)]
    ly = [torch.empty(1024, dtype=torch.float32, device="cuda") for _ in range(3)]
    ops.append(("gemv layers", lambda: q4k.gemv_layers(lw, lx, ly), ly, True))

    torch.cuda.synchronize()
    eager = []
    for name, run, outs, _ in ops:
        run()
        torch.cuda.synchronize()
        eager.append([t.clone() for t in outs])

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, run, _, _ in ops:
            run()
    torch.cuda.synchronize()

    for replay in range(3):
        for _, _, outs, _ in ops:
            for t in outs:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (name, _, outs, exact), ref in zip(ops, eager):
            for t, r in zip(outs, ref):
                if exact:
                    assert torch.equal(t.view(torch.int32), r.view(torch.int32)), \
                        "%s: replay %d differs from the eager run" % (name, replay)
                else:
                    assert torch.isfinite(t).all(), "%s: replay %d left NaN" % (name, replay)
                    tol = 1e-5 * r.abs().max().item() + 1e-30
                    diff = (t - r).abs().max().item()
                    assert diff <= tol, "%s: replay %d off by %g" % (name, replay, diff)


def test_graph_split_k_replay_matches_oracle(q4k):
    # Split K zeroes its output with a kernel inside the graph; a replay over
    # NaN-filled output must still give the oracle's result.
    m, n, k = 64, 4000, 2048
    w = synth.q4k_weights(n, k, seed=9)
    xb = synth.normal_bf16((m, k), seed=9)
    wd, xd = dev(w), dev_bf16(xb)
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    q4k.gemm(wd, xd, out=y)  # warm-up outside capture
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        q4k.gemm(wd, xd, out=y)
    cols = np.arange(0, n, 97)
    Yr, A = oracle.gemm_cols(w, xb, n, k, cols)
    for _ in range(2):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y.cpu().numpy()[:, cols].astype(np.float64)
        assert np.all(np.abs(got - Yr) <= 1e-2 * A)


def test_graph_sibling_formats_and_w8a8_replay(q4k):
    # The other families under capture: the split-bf16 MFMA GEMV, the Q5_K, Q6_K and
    # Q3_K GEMVs (batched passes), their LDS-dequant GEMMs (split K with its
    # zeroing kernel, and without), the dequant exports, and the INT8 layer and
    # row quantizer.  Outputs allocated inside the capture live in the graph's
    # pool and are rewritten by every replay.
    ops = []  # (name, outputs, exact)
    caps = []  # run() -> outputs, called once eagerly and once under capture

    def add(name, run, exact=True):
        caps.append((name, run, exact))

    n, k = 2048, 1024
    for fmt, gen, gv in (("q4k", synth.q4k_weights, q4k.gemv), ("q5k", synth.q5k_weights, q4k.q5k_gemv),
                         ("q6k", synth.q6k_weights, q4k.q6k_gemv), ("q3k", synth.q3k_weights, q4k.q3k_gemv)):
        w = dev(gen(n, k, seed=61))
        for m in (1, 6, 9):
            x = dev(synth.normal_f32((m, k), seed=60 + m))
            add("%s gemv m=%d" % (fmt, m), lambda w=w, x=x, gv=gv: [gv(w, x)])
    for fmt, gen, gm in (("q5k", synth.q5k_weights, q4k.q5k_gemm), ("q6k", synth.q6k_weights, q4k.q6k_gemm),
                         ("q3k", synth.q3k_weights, q4k.q3k_gemm)):
        # split K; full grid; a small batch on a wide matrix (Q5_K: the streaming kernel)
        for m, nn, kk in ((64, 1000, 1024), (300, 4096, 512), (16, 8192, 512)):
            w = dev(gen(nn, kk, seed=m))
            xb = dev_bf16(synth.normal_bf16((m, kk), seed=m))
            add("%s gemm %dx%dx%d" % (fmt, m, nn, kk), lambda w=w, xb=xb, gm=gm: [gm(w, xb)],
                exact=m == 300 or (fmt == "q5k" and m == 16))
    for fmt, gen, dq in (("q6k", synth.q6k_weights, q4k.q6k_dequantize_bf16),
                         ("q3k", synth.q3k_weights, q4k.q3k_dequantize_f32)):
        w = dev(gen(256, 512, seed=3))
        add("%s dequant" % fmt, lambda w=w, dq=dq: [dq(w)])
    # the INT8 layer's tile shapes: 64 x 64, 64 x 192 (three-slot ring), 128 x 192
    for m8, n8, k8 in ((256, 512, 1024), (1030, 3072, 256), (2200, 1920, 256)):
        x8, xs, w8, ws, b = (dev(a) for a in synth.w8a8_case(m8, n8, k8, seed=5))
        add("w8a8_linear %dx%dx%d" % (m8, n8, k8),
            lambda x8=x8, xs=xs, w8=w8, ws=ws, b=b: [q4k.w8a8_linear(x8, xs, w8, ws, b)])
    xq = dev_bf16(synth.normal_bf16((64, 1024), seed=5))
    add("w8a8_quantize_rows", lambda: list(q4k.w8a8_quantize_rows(xq)))

    torch.cuda.synchronize()
    eager = []
    for name, run, _ in caps:
        eager.append([t.clone() for t in run()])
        torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    outs = []
    with torch.cuda.graph(g):
        for name, run, exact in caps:
            outs.append(run())
    torch.cuda.synchronize()

    for replay in range(3):
        for o in outs:
            for t in o:
                t.zero_() if not t.is_floating_point() else t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (name, _, exact), o, ref in zip(caps, outs, eager):
            for t, r in zip(o, ref):
                if exact or not t.is_floating_point():
                    assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), \
                        "%s: replay %d differs from the eager run" % (name, replay)
                else:
                    assert torch.isfinite(t).all(), "%s: replay %d left NaN" % (name, replay)
                    tol = 1e-5 * r.abs().max().item() + 1e-30
                    diff = (t - r).abs().max().item()
                    assert diff <= tol, "%s: replay %d off by %g" % (name, replay, diff)
